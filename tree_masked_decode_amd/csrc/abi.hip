// abi.hip -- the extern "C" entry points of libtreeattn.so: argument and
// buffer validation, launch planning and kernel dispatch.
//
// Validation follows "ops/tree_attention.rs" (mlx-native 0.9.2),
// validate_params and validate_buffers: supported head dims, head counts
// and divisibility, kv_seq_len / kv_capacity / q_l / mask_stride rules, and
// byte-size checks done with overflow-checked arithmetic so that a huge
// shape cannot wrap into a small requirement.  Every check runs before any
// HIP call; a failing call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include "../../include/tree_attn.h"
#include "common.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return TA_OK;
}

// Overflow-checked products.
bool mul_ok(uint64_t a, uint64_t b, uint64_t &r) {
  if (a != 0 && b > UINT64_MAX / a) return false;
  r = a * b;
  return true;
}
bool mul3(uint64_t a, uint64_t b, uint64_t c, uint64_t &r) {
  uint64_t t;
  return mul_ok(a, b, t) && mul_ok(t, c, r);
}
bool mul4(uint64_t a, uint64_t b, uint64_t c, uint64_t d, uint64_t &r) {
  uint64_t t;
  return mul3(a, b, c, t) && mul_ok(t, d, r);
}
bool add_ok(uint64_t a, uint64_t b, uint64_t &r) {
  if (b > UINT64_MAX - a) return false;
  r = a + b;
  return true;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// One argument rule: when `bad`, the call fails with `code` and the message
// fmt (fn, a, b) -- two unsigned numbers at most, formatted only on failure.
struct Rule {
  bool bad;
  int code;
  const char *fmt;
  unsigned long long a, b;
};

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return fail(TA_EHIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Largest split count accepted (keeps every grid dimension and index in
// range; far beyond any useful value).
constexpr uint32_t kMaxNwg = 65536;
// Key ranges of the live-key scan (8 bytes of result each).
constexpr uint32_t kRangeChunks = TA_RANGE_BYTES / 8;
static_assert(TA_RANGE_BYTES % 8 == 0, "range chunks");

uint64_t partials_bytes_u64(uint64_t nrows, uint64_t dim, uint64_t nwg,
                            bool &overflow) {
  uint64_t r;
  overflow = !mul4(nrows, nwg, dim + 2, 4, r);
  return overflow ? UINT64_MAX : r;
}

// Split count for `heads` independent (kv head) streams of `row_tiles`
// workgroups each.  Workgroup ids go to the 8 XCDs in turn and every row tile
// of one (head, split) unit sits on one XCD, so an XCD holds
// ceil(heads * nwg / 8) * row_tiles workgroups: as many splits as keep that
// within ONE round of the XCD's resident slots (CUs per XCD * per_cu), with at
// least min_tiles key tiles per split and partial-result bytes (written once,
// read once by the merge) of at most 2/5 of the K/V bytes.  (The cap bites on
// short calls: a 17 MB tree measured 27.0-28.4 us per call from 16 to 42
// splits while its partials grew 2.6 times; the 32K tree's 32 splits write 38%
// of its K/V bytes.)
uint32_t pick_splits(uint32_t heads, uint32_t row_tiles, uint32_t n_tiles, uint32_t num_cus,
                     uint32_t per_cu, uint32_t min_tiles, uint64_t kv_bytes,
                     uint64_t partial_bytes_per_split) {
  if (num_cus == 0) num_cus = 256;
  const uint64_t slots_per_xcd = (uint64_t)(num_cus / ta::kXcds) * per_cu;
  const uint64_t units_per_xcd = row_tiles ? slots_per_xcd / row_tiles : 0;
  uint64_t nwg = units_per_xcd * ta::kXcds / heads;
  const uint64_t by_tiles = n_tiles / min_tiles;
  if (nwg > by_tiles) nwg = by_tiles;
  if (partial_bytes_per_split > 0 && nwg > kv_bytes * 2 / 5 / partial_bytes_per_split)
    nwg = kv_bytes * 2 / 5 / partial_bytes_per_split;
  if (nwg < 1) nwg = 1;
  if (nwg > kMaxNwg) nwg = kMaxNwg;
  return (uint32_t)nwg;
}

}  // namespace

// Split partials of tree_attn_forward_noalloc: one buffer per GPU, part of
// this file's device code object (so it exists on every device the library
// runs on, for the life of the process).  Host code never uses this name for
// the memory: on the host it only names a stand-in.  The device address comes
// from the runtime, once per device (static_scratch).
constexpr uint64_t kStaticScratchBytes = TA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch_dev[kMaxDevices];  // zero-initialised (static storage)

// Device address of `scratch` on the device of stream `s` (the current device
// for the null stream), looked up on the first call for that device with the
// device current.  nullptr (and the error string set) on failure.
float *static_scratch(const char *fn, hipStream_t s) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(TA_EHIP, "%s: cannot find the stream's device: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(TA_EHIP, "%s: device ordinal %d beyond the %d the library tracks", fn, dev,
         kMaxDevices);
    return nullptr;
  }
  float *p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (p) return p;
  int cur = -1;
  e = hipGetDevice(&cur);
  if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
  void *addr = nullptr;
  hipError_t el = e == hipSuccess ? hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) : e;
  if (e == hipSuccess && cur != dev) e = hipSetDevice(cur);
  if (el != hipSuccess || e != hipSuccess || addr == nullptr) {
    fail(TA_EHIP, "%s: cannot find the static scratch on device %d: %s", fn, dev,
         hipGetErrorString(el != hipSuccess ? el : e));
    return nullptr;
  }
  // (two threads racing here both store the same address)
  g_scratch_dev[dev].store(static_cast<float *>(addr), std::memory_order_release);
  return static_cast<float *>(addr);
}

}  // namespace

extern "C" {

const char *tree_attn_last_error(void) { return g_err.c_str(); }

size_t tree_attn_partials_bytes(uint32_t n_heads, uint32_t head_dim,
                                uint32_t q_l, uint32_t nwg) {
  bool of;
  uint64_t r = partials_bytes_u64((uint64_t)n_heads * q_l, head_dim, nwg, of);
  if (of || r > (uint64_t)SIZE_MAX) return SIZE_MAX;
  return (size_t)r;
}

uint32_t tree_attn_pick_nwg(uint32_t n_heads, uint32_t n_kv_heads,
                            uint32_t head_dim, uint32_t kv_seq_len,
                            uint32_t q_l, int kv_dtype, uint32_t num_cus) {
  if (n_heads == 0 || n_kv_heads == 0 || kv_seq_len == 0 || q_l == 0 ||
      n_heads % n_kv_heads != 0)
    return 1;
  uint32_t rows = q_l * (n_heads / n_kv_heads);
  bool f16 = kv_dtype == TA_F16;
  // (the planner assumes a 16-byte aligned mask with a stride of whole
  // 16-byte chunks, or none)
  uint32_t rpw = f16 ? ta::f16_rows_per_wg(head_dim, rows, n_heads / n_kv_heads, false, true)
                     : ta::kF32RowsPerWG;
  uint32_t bn = f16 ? ta::f16_tile_keys(head_dim) : ta::f32_tile_keys(head_dim);
  // One resident fp16 workgroup per CU (its registers fill the SIMDs); the
  // fp32 kernel fits two.
  uint32_t per_cu = f16 ? 1u : 2u;
  const uint64_t kv = 2ull * n_kv_heads * kv_seq_len * head_dim * (f16 ? 2u : 4u);
  const uint64_t part = (uint64_t)n_heads * q_l * (head_dim + 2) * 4;
  return pick_splits(n_kv_heads, ceil_div(rows, rpw), ceil_div(kv_seq_len, bn), num_cus,
                     per_cu, 2u, kv, part);
}

uint32_t tree_attn_quant_pick_nwg(uint32_t batch, uint32_t n_q_heads,
                                  uint32_t n_kv_heads, uint32_t dim,
                                  uint32_t kv_seq_len, uint32_t q_l,
                                  uint32_t num_cus) {
  if (batch == 0 || n_q_heads == 0 || n_kv_heads == 0 || kv_seq_len == 0 ||
      q_l == 0 || n_q_heads % n_kv_heads != 0)
    return 1;
  uint32_t rows = q_l * (n_q_heads / n_kv_heads);
  // one-wavefront workgroups, several resident per CU
  const uint64_t kv = 2ull * batch * n_kv_heads * kv_seq_len * dim / 2;
  const uint64_t part = (uint64_t)batch * n_q_heads * q_l * (dim + 2) * 4;
  return pick_splits(batch * n_kv_heads, ceil_div(rows, ta::kQuantRowsPerWG),
                     ceil_div(kv_seq_len, ta::quant_tile_keys(dim)), num_cus, 8u, 2u, kv, part);
}

static int fp_forward(const char *fn, const float *q, size_t q_bytes, const void *k,
                      const void *v, int kv_dtype, size_t kv_bytes,
                      const float *mask, size_t mask_bytes, float *partials,
                      size_t partials_bytes, float *out, size_t out_bytes,
                      uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                      uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
                      uint32_t mask_stride, uint32_t window_start, float scale,
                      uint32_t nwg, void *stream, bool static_partials = false) {
  // Checked in table order; the first rule that fails names the problem
  // and nothing is launched.  The contract (head dims, GQA divisibility,
  // capacity, mask stride, byte sizes with checked products) is the one
  // "ops/tree_attention.rs" states in validate_params and validate_buffers.
  const bool f16 = kv_dtype == TA_F16;
  const Rule args[] = {
      {!q || !k || !v, TA_EINVAL, "%s: a NULL pointer among q, k, v", 0, 0},
      {nwg == 1 && !out, TA_EINVAL, "%s: one split writes the result: out is NULL", 0, 0},
      {nwg > 1 && !partials && !static_partials, TA_EINVAL,
       "%s: %llu splits write partial results: partials is NULL", nwg, 0},
      {kv_dtype != TA_F32 && kv_dtype != TA_F16, TA_EUNSUPPORTED,
       "%s: unknown k/v dtype code %lld (TA_F32 or TA_F16)", (unsigned long long)(int64_t)kv_dtype,
       0},
      {head_dim != 128 && head_dim != 256 && head_dim != 512, TA_EUNSUPPORTED,
       "%s: head_dim %llu not built (128, 256 and 512 are)", head_dim, 0},
      {n_heads == 0, TA_EINVAL, "%s: n_heads is 0", 0, 0},
      {n_kv_heads == 0, TA_EINVAL, "%s: n_kv_heads is 0", 0, 0},
      {n_kv_heads != 0 && n_heads % n_kv_heads != 0, TA_EINVAL,
       "%s: n_heads %llu is not a multiple of n_kv_heads %llu", n_heads, n_kv_heads},
      {q_l == 0, TA_EINVAL, "%s: q_l (tree nodes) is 0", 0, 0},
      {kv_seq_len == 0, TA_EINVAL, "%s: kv_seq_len is 0", 0, 0},
      {kv_capacity < kv_seq_len, TA_EINVAL, "%s: kv_capacity %llu holds fewer than kv_seq_len %llu keys",
       kv_capacity, kv_seq_len},
      {mask != nullptr && mask_stride < kv_seq_len, TA_EINVAL,
       "%s: mask_stride %llu is shorter than kv_seq_len %llu", mask_stride, kv_seq_len},
      {kv_seq_len != 0 && window_start >= kv_seq_len, TA_EINVAL,
       "%s: window_start %llu leaves no key (kv_seq_len %llu)", window_start, kv_seq_len},
      {nwg == 0 || nwg > kMaxNwg, TA_EINVAL, "%s: nwg %llu outside [1, %llu]", nwg, kMaxNwg},
      {!(scale == scale) || scale == INFINITY || scale == -INFINITY, TA_EINVAL,
       "%s: scale is not a finite number", 0, 0},
      {!aligned16(q) || !aligned16(k) || !aligned16(v) || (out && !aligned16(out)) ||
           (partials && !aligned16(partials)) || (mask && ((uintptr_t)mask & 3u)),
       TA_EINVAL, "%s: device pointers must be 16-byte aligned (the mask 4-byte aligned)", 0, 0},
  };
  for (const Rule &r : args)
    if (r.bad) return fail(r.code, r.fmt, fn, r.a, r.b);

  // bytes each buffer must hold (64-bit products, overflow checked)
  const uint64_t esz = f16 ? 2 : 4;
  uint64_t req_q, req_kv, req_mask = 0, req_part = 0;
  bool of = !mul4(n_heads, q_l, head_dim, 4, req_q) ||
            !mul4(n_kv_heads, kv_capacity, head_dim, esz, req_kv) ||
            (mask && !mul3(q_l, mask_stride, 4, req_mask));
  if (nwg > 1 && !of) {
    bool pof;
    req_part = partials_bytes_u64((uint64_t)n_heads * q_l, head_dim, nwg, pof);
    of = pof;
  }
  if (of) return fail(TA_EOVERFLOW, "%s: a buffer size overflows 64 bits", fn);
  const uint64_t req_out = req_q;   // out holds as many floats as q
  const Rule sizes[] = {
      {q_bytes < req_q, TA_ESIZE, "%s: q buffer holds %llu bytes of the %llu needed", q_bytes,
       req_q},
      {kv_bytes < req_kv, TA_ESIZE, "%s: k/v buffers hold %llu bytes of the %llu needed", kv_bytes,
       req_kv},
      {mask && mask_bytes < req_mask, TA_ESIZE,
       "%s: tree mask holds %llu bytes of the %llu needed", mask_bytes, req_mask},
      {nwg == 1 && out_bytes < req_out, TA_ESIZE,
       "%s: output buffer holds %llu bytes of the %llu needed", out_bytes, req_out},
      {static_partials && req_part > kStaticScratchBytes, TA_ESIZE,
       "%s: partials of these splits need %llu bytes, the static scratch holds %llu: use fewer "
       "splits",
       req_part, kStaticScratchBytes},
      {!static_partials && nwg > 1 && partials_bytes < req_part, TA_ESIZE,
       "%s: partials buffer holds %llu bytes of the %llu needed", partials_bytes, req_part},
  };
  for (const Rule &r : sizes)
    if (r.bad) return fail(r.code, r.fmt, fn, r.a, r.b);
  // row count per kv head and the grid must fit the kernels' 32-bit indices
  uint64_t rows = (uint64_t)q_l * (n_heads / n_kv_heads);
  if ((uint64_t)n_heads * q_l > 0x7fffffffull || rows > 0x7fffffffull)
    return fail(TA_EUNSUPPORTED, "%s: n_heads*q_l too large", fn);

  // --- plan and launch ---
  ta::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.mask = mask;
  a.out = out;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.group = n_heads / n_kv_heads;
  a.kv_seq_len = kv_seq_len;
  a.kv_capacity = kv_capacity;
  a.q_l = q_l;
  a.mask_stride = mask ? mask_stride : kv_seq_len;
  a.nwg = nwg;
  a.rows = (uint32_t)rows;
  a.key_lo = mask ? 0u : window_start;
  a.qscale = scale * ta::kLog2e;
  a.scale = scale;
  const bool mask_vec = mask == nullptr || ((uintptr_t)mask % 16u == 0 && mask_stride % 4u == 0);
  const uint32_t rpw = f16 ? ta::f16_rows_per_wg(head_dim, a.rows, a.group, mask == nullptr, mask_vec)
                           : ta::kF32RowsPerWG;
  const uint32_t bn = f16 ? ta::f16_tile_keys(head_dim) : ta::f32_tile_keys(head_dim);
  a.row_tiles = ceil_div(a.rows, rpw);
  a.n_tiles = ceil_div(kv_seq_len, bn);
  uint64_t units = (uint64_t)n_kv_heads * nwg;
  uint64_t blocks = (uint64_t)ta::kXcds * ((units + ta::kXcds - 1) / ta::kXcds) * a.row_tiles;
  if (blocks > 0x7fffffffull)
    return fail(TA_EUNSUPPORTED, "%s: grid too large (n_kv_heads*nwg*row tiles)", fn);
  a.units = (uint32_t)units;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (static_partials && nwg > 1) {
    partials = static_scratch(fn, s);
    if (!partials) return TA_EHIP;
  }
  if (nwg > 1) {
    a.part_o = partials;
    a.part_sm = partials + (size_t)nwg * n_heads * q_l * head_dim;
  } else {
    a.part_o = a.part_sm = nullptr;
  }
  // Live-key scan of an explicit mask, into the TA_RANGE_BYTES after the
  // partials when the buffer holds them.  Worth one more launch only where
  // the K/V stream is long (>= 64 MiB) and the mask is small beside it
  // (<= 1/32 of it): a dead prefix or suffix then costs neither fetches nor
  // idle splits; shorter calls would mostly pay the extra launch.
  a.range = nullptr;
  a.range_chunks = 0;
  const uint64_t spare =
      static_partials ? kStaticScratchBytes - req_part : (uint64_t)partials_bytes - req_part;
  const uint64_t kv_read = 2ull * n_kv_heads * kv_seq_len * head_dim * esz;
  const uint64_t mask_read = (uint64_t)q_l * kv_seq_len * 4u;
  if (mask && nwg > 1 && spare >= TA_RANGE_BYTES && kv_read >= (64ull << 20) &&
      kv_read >= 32u * mask_read) {
    ta::MaskRangeArgs r;
    r.mask = mask;
    r.out = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(partials) + req_part);
    r.q_l = q_l;
    r.kv_seq_len = kv_seq_len;
    r.mask_stride = mask_stride;
    r.chunks = kv_seq_len < kRangeChunks ? kv_seq_len : kRangeChunks;
    hipError_t er = ta::launch_mask_range(r, s);
    if (er != hipSuccess) return hip_status(er, fn);
    a.range = r.out;
    a.range_chunks = r.chunks;
  }
  // Non-temporal K/V copies for long streams: the 128K chain measured 392
  // -> 352 us per call with them, a 17 MB tree 22.5 -> 23.9 us forward.
  a.stream_nt = kv_read >= (64ull << 20) ? 1u : 0u;
  hipError_t e = f16 ? ta::launch_forward_f16(a, head_dim, s)
                     : ta::launch_forward_f32(a, head_dim, s);
  return hip_status(e, fn);
}

uint32_t tree_attn_quant_pick_nwg_ex(uint32_t batch, uint32_t n_q_heads,
                                     uint32_t n_kv_heads, uint32_t dim,
                                     uint32_t kv_seq_len, uint32_t q_l, uint32_t bits,
                                     uint32_t group_size, int mask_kind, int q_dtype,
                                     uint32_t num_cus) {
  if (batch == 0 || n_q_heads == 0 || n_kv_heads == 0 || kv_seq_len == 0 ||
      q_l == 0 || n_q_heads % n_kv_heads != 0)
    return 1;
  const int elem = q_dtype == TA_BF16 ? 1 : q_dtype == TA_F32 ? 2 : 0;
  uint32_t per_cu = ta::quant_wgs_per_cu(dim, bits, group_size, mask_kind, elem);
  // Not a supported variant: the plain estimate.  Beyond two wavefronts per
  // SIMD the four SIMDs of a CU no longer get equal shares (10 workgroups
  // put three on two of them), which measured slower than 8.
  if (per_cu == 0 || per_cu > 8u) per_cu = 8u;
  uint32_t rows = q_l * (n_q_heads / n_kv_heads);
  const uint64_t kv = 2ull * batch * n_kv_heads * kv_seq_len * dim * (bits ? bits : 4) / 8;
  const uint64_t part = (uint64_t)batch * n_q_heads * q_l * (dim + 2) * 4;
  return pick_splits(batch * n_kv_heads, ceil_div(rows, ta::kQuantRowsPerWG),
                     ceil_div(kv_seq_len, ta::quant_tile_keys(dim)), num_cus, per_cu, 2u, kv,
                     part);
}

int tree_attn_forward(const float *q, size_t q_bytes, const void *k,
                      const void *v, int kv_dtype, size_t kv_bytes,
                      const float *mask, size_t mask_bytes, float *partials,
                      size_t partials_bytes, float *out, size_t out_bytes,
                      uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                      uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
                      uint32_t mask_stride, float scale, uint32_t nwg,
                      void *stream) {
  return fp_forward("tree_attn_forward", q, q_bytes, k, v, kv_dtype, kv_bytes, mask,
                    mask_bytes, partials, partials_bytes, out, out_bytes, n_heads,
                    n_kv_heads, head_dim, kv_seq_len, kv_capacity, q_l, mask_stride, 0u,
                    scale, nwg, stream);
}

int tree_attn_decode(const float *q, size_t q_bytes, const void *k, const void *v,
                     int kv_dtype, size_t kv_bytes, float *partials,
                     size_t partials_bytes, float *out, size_t out_bytes,
                     uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                     uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
                     uint32_t window_start, float scale, uint32_t nwg, void *stream) {
  return fp_forward("tree_attn_decode", q, q_bytes, k, v, kv_dtype, kv_bytes, nullptr, 0,
                    partials, partials_bytes, out, out_bytes, n_heads, n_kv_heads,
                    head_dim, kv_seq_len, kv_capacity, q_l, kv_seq_len, window_start, scale,
                    nwg, stream);
}

int tree_attn_reduce(const float *partials, size_t partials_bytes, void *out,
                     int out_dtype, size_t out_bytes, uint32_t nrows,
                     uint32_t head_dim, uint32_t nwg, void *stream) {
  const char *fn = "tree_attn_reduce";
  if (nrows == 0) return fail(TA_EINVAL, "%s: nrows must be > 0", fn);
  if (head_dim == 0 || head_dim % 4 != 0 || head_dim > 512)
    return fail(TA_EUNSUPPORTED, "%s: head_dim must be a multiple of 4 in [4, 512], got %u",
                fn, head_dim);
  if (nwg == 0 || nwg > kMaxNwg)
    return fail(TA_EINVAL, "%s: nwg must be in [1, %u], got %u", fn, kMaxNwg, nwg);
  if (out_dtype != TA_F32 && out_dtype != TA_F16 && out_dtype != TA_BF16)
    return fail(TA_EUNSUPPORTED, "%s: out dtype must be TA_F32, TA_F16 or TA_BF16", fn);
  if (!partials || !out) return fail(TA_EINVAL, "%s: partials and out must not be NULL", fn);
  if (!aligned16(partials) || ((uintptr_t)out & 7u))
    return fail(TA_EINVAL, "%s: partials must be 16-byte and out 8-byte aligned", fn);
  bool of;
  uint64_t req_part = partials_bytes_u64(nrows, head_dim, nwg, of);
  uint64_t req_out;
  if (of || !mul3(nrows, head_dim, out_dtype == TA_F32 ? 4 : 2, req_out))
    return fail(TA_EOVERFLOW, "%s: size computation overflows", fn);
  if (partials_bytes < req_part)
    return fail(TA_ESIZE, "%s: partials buffer holds %zu bytes of the %llu needed",
                fn, partials_bytes, (unsigned long long)req_part);
  if (out_bytes < req_out)
    return fail(TA_ESIZE, "%s: output buffer holds %zu bytes of the %llu needed", fn,
                out_bytes, (unsigned long long)req_out);
  if (nrows > 0x7ffffff0u) return fail(TA_EUNSUPPORTED, "%s: nrows too large", fn);
  ta::ReduceArgs a;
  a.part_o = partials;
  a.part_sm = partials + (size_t)nwg * nrows * head_dim;
  a.out = out;
  a.nrows = nrows;
  a.dim = head_dim;
  a.nwg = nwg;
  a.out_type = out_dtype == TA_F16 ? 1 : out_dtype == TA_BF16 ? 2 : 0;
  return hip_status(ta::launch_reduce(a, static_cast<hipStream_t>(stream)), fn);
}

int tree_attn_forward_noalloc(const float *q, size_t q_bytes, const void *k, const void *v,
                              int kv_dtype, size_t kv_bytes, const float *mask,
                              size_t mask_bytes, float *out, size_t out_bytes, uint32_t n_heads,
                              uint32_t n_kv_heads, uint32_t head_dim, uint32_t kv_seq_len,
                              uint32_t kv_capacity, uint32_t q_l, uint32_t mask_stride,
                              float scale, uint32_t nwg, void *stream) {
  const char *fn = "tree_attn_forward_noalloc";
  if (!out) return fail(TA_EINVAL, "%s: out must not be NULL", fn);
  // the forward validates everything (the split results' size against the
  // static scratch included), then looks the scratch up and launches
  int rc = fp_forward(fn, q, q_bytes, k, v, kv_dtype, kv_bytes, mask, mask_bytes, nullptr, 0,
                      out, out_bytes, n_heads, n_kv_heads, head_dim, kv_seq_len, kv_capacity,
                      q_l, mask_stride, 0u, scale, nwg, stream, true);
  if (rc != TA_OK || nwg == 1) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *part = static_scratch(fn, s);
  if (!part) return TA_EHIP;
  const uint32_t nrows = n_heads * q_l;  // < 2^31: checked by the forward
  ta::ReduceArgs a;
  a.part_o = part;
  a.part_sm = part + (size_t)nwg * nrows * head_dim;
  a.out = out;
  a.nrows = nrows;
  a.dim = head_dim;
  a.nwg = nwg;
  a.out_type = 0;
  return hip_status(ta::launch_reduce(a, s), fn);
}

static int quant_forward(
    const char *fn, const void *q, int q_dtype, size_t q_bytes, const uint32_t *k_packed,
    const void *k_scales, const void *k_biases, const uint32_t *v_packed,
    const void *v_scales, const void *v_biases, const size_t kv_bytes[6],
    const float *sinks, size_t sinks_bytes, const void *mask, int mask_kind,
    size_t mask_bytes, uint64_t mask_head_stride, uint32_t mask_stride,
    uint32_t window_size, float *partials, size_t partials_bytes, void *out,
    size_t out_bytes, uint32_t batch, uint32_t n_q_heads, uint32_t n_kv_heads,
    uint32_t dim, uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
    uint32_t bits, uint32_t group_size, float scale, uint32_t nwg, void *stream) {
  if (mask_kind != TA_MASK_NONE && mask_kind != TA_MASK_F16 && mask_kind != TA_MASK_BOOL)
    return fail(TA_EINVAL, "%s: mask_kind must be TA_MASK_NONE, TA_MASK_F16 or TA_MASK_BOOL",
                fn);
  if ((mask_kind == TA_MASK_NONE) != (mask == nullptr))
    return fail(TA_EINVAL, "%s: mask must be NULL exactly when mask_kind is TA_MASK_NONE", fn);
  if (q_dtype != TA_F16 && q_dtype != TA_BF16 && q_dtype != TA_F32)
    return fail(TA_EUNSUPPORTED,
                "%s: queries/scales/biases/mask/out dtype must be TA_F16, TA_BF16 or TA_F32", fn);
  const uint64_t esz = q_dtype == TA_F32 ? 4 : 2;   // bytes of a T element
  const uint64_t cell_bytes = mask_kind == TA_MASK_BOOL ? 4 : esz;
  if (bits != 4 && bits != 8)
    return fail(TA_EUNSUPPORTED, "%s: bits must be 4 or 8, got %u", fn, bits);
  if (dim != 64 && dim != 96 && dim != 128 && dim != 256 && dim != 512)
    return fail(TA_EUNSUPPORTED, "%s: dim must be 64, 96, 128, 256 or 512, got %u", fn, dim);
  if (group_size != 32 && group_size != 64 && group_size != 128)
    return fail(TA_EUNSUPPORTED, "%s: group_size must be 32, 64 or 128, got %u", fn,
                group_size);
  if (dim % group_size != 0)
    return fail(TA_EINVAL, "%s: dim (%u) must be divisible by group_size (%u)", fn, dim,
                group_size);
  if (batch == 0 || n_q_heads == 0 || n_kv_heads == 0)
    return fail(TA_EINVAL, "%s: batch, n_q_heads and n_kv_heads must be > 0", fn);
  if (n_q_heads % n_kv_heads != 0)
    return fail(TA_EINVAL, "%s: n_q_heads (%u) must be divisible by n_kv_heads (%u)", fn,
                n_q_heads, n_kv_heads);
  if (kv_seq_len == 0) return fail(TA_EINVAL, "%s: kv_seq_len must be > 0", fn);
  if (kv_capacity < kv_seq_len)
    return fail(TA_EINVAL, "%s: kv_capacity %u holds fewer than kv_seq_len %u keys", fn,
                kv_capacity, kv_seq_len);
  if (q_l == 0) return fail(TA_EINVAL, "%s: q_seq_len (q_l) must be > 0", fn);
  if (mask != nullptr && mask_stride < kv_seq_len)
    return fail(TA_EINVAL, "%s: mask_stride %u is shorter than kv_seq_len %u", fn,
                mask_stride, kv_seq_len);
  if (nwg == 0 || nwg > kMaxNwg)
    return fail(TA_EINVAL, "%s: nwg must be in [1, %u], got %u", fn, kMaxNwg, nwg);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(TA_EINVAL, "%s: scale must be finite", fn);
  // Scales/biases are read four tokens at a time as 32-bit words: a head's
  // block of them (kv_capacity tokens of (dim/group_size) T each) must start
  // on a 4-byte boundary, which an odd capacity breaks whenever one token's
  // scales fill an odd number of 2-byte elements.
  if ((dim / group_size) * esz % 4 != 0 && (kv_capacity & 1u))
    return fail(TA_EUNSUPPORTED,
                "%s: kv_capacity must be even when dim/group_size is odd with 2-byte scales",
                fn);
  if (!kv_bytes) return fail(TA_EINVAL, "%s: kv_bytes must not be NULL", fn);
  if (!q || !k_packed || !k_scales || !k_biases || !v_packed || !v_scales || !v_biases)
    return fail(TA_EINVAL, "%s: q and the six K/V buffers must not be NULL", fn);
  if (nwg == 1 && !out) return fail(TA_EINVAL, "%s: out must not be NULL when nwg == 1", fn);
  if (nwg > 1 && !partials)
    return fail(TA_EINVAL, "%s: partials must not be NULL when nwg > 1", fn);
  const void *ptrs[] = {q, k_packed, k_scales, k_biases, v_packed, v_scales, v_biases};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(TA_EINVAL, "%s: device pointers must be 16-byte aligned", fn);
  if ((out && !aligned16(out)) || (partials && !aligned16(partials)) ||
      (mask && ((uintptr_t)mask & (cell_bytes - 1))) || (sinks && ((uintptr_t)sinks & 3u)))
    return fail(TA_EINVAL, "%s: device pointers must be 16-byte aligned", fn);

  const uint64_t BnQ = (uint64_t)batch * n_q_heads, BnKV = (uint64_t)batch * n_kv_heads;
  const uint64_t pf = 32 / bits;
  uint64_t req_q, req_packed, req_sb, req_out, req_sinks = 0, req_mask = 0, req_part = 0;
  if (!mul4(BnQ, q_l, dim, esz, req_q) || !mul4(BnKV, kv_capacity, dim / pf, 4, req_packed) ||
      !mul4(BnKV, kv_capacity, dim / group_size, esz, req_sb))
    return fail(TA_EOVERFLOW, "%s: size computation overflows", fn);
  req_out = req_q;
  if (sinks) req_sinks = (uint64_t)n_q_heads * 4;
  if (mask) {
    // last cell: (BnQ-1)*mask_head_stride + (q_l-1)*mask_stride + (kv_seq_len-1)
    uint64_t t1, t2, t3;
    if (!mul_ok(BnQ - 1, mask_head_stride, t1) || !mul_ok(q_l - 1, mask_stride, t2) ||
        !add_ok(t1, t2, t3) || !add_ok(t3, kv_seq_len, t3) || !mul_ok(t3, cell_bytes, req_mask))
      return fail(TA_EOVERFLOW, "%s: mask extent overflows", fn);
  }
  bool of = false;
  if (nwg > 1) req_part = partials_bytes_u64(BnQ * q_l, dim, nwg, of);
  if (of) return fail(TA_EOVERFLOW, "%s: partials size overflows", fn);
  if (q_bytes < req_q)
    return fail(TA_ESIZE, "%s: q buffer holds %zu bytes of the %llu needed", fn, q_bytes,
                (unsigned long long)req_q);
  const char *names[6] = {"k_packed", "k_scales", "k_biases", "v_packed", "v_scales", "v_biases"};
  for (int b = 0; b < 6; ++b) {
    uint64_t need = (b % 3 == 0) ? req_packed : req_sb;
    if (kv_bytes[b] < need)
      return fail(TA_ESIZE, "%s: %s buffer holds %zu bytes of the %llu needed", fn,
                  names[b], kv_bytes[b], (unsigned long long)need);
  }
  if (sinks && sinks_bytes < req_sinks)
    return fail(TA_ESIZE, "%s: sinks buffer holds %zu bytes of the %llu needed", fn,
                sinks_bytes, (unsigned long long)req_sinks);
  if (mask && mask_bytes < req_mask)
    return fail(TA_ESIZE, "%s: mask buffer holds %zu bytes of the %llu needed", fn,
                mask_bytes, (unsigned long long)req_mask);
  if (nwg == 1 && out_bytes < req_out)
    return fail(TA_ESIZE, "%s: output buffer holds %zu bytes of the %llu needed", fn,
                out_bytes, (unsigned long long)req_out);
  if (nwg > 1 && partials_bytes < req_part)
    return fail(TA_ESIZE, "%s: partials buffer holds %zu bytes of the %llu needed", fn,
                partials_bytes, (unsigned long long)req_part);
  uint64_t rows = (uint64_t)q_l * (n_q_heads / n_kv_heads);
  if (BnQ * q_l > 0x7fffffffull || rows > 0x7fffffffull)
    return fail(TA_EUNSUPPORTED, "%s: batch*n_q_heads*q_l too large", fn);

  ta::QuantArgs a;
  a.q = q;
  a.elem = q_dtype == TA_BF16 ? 1 : q_dtype == TA_F32 ? 2 : 0;
  a.kp = k_packed;
  a.vp = v_packed;
  a.ks = k_scales;
  a.kb = k_biases;
  a.vs = v_scales;
  a.vb = v_biases;
  a.sinks = sinks;
  a.mask = mask_kind == TA_MASK_F16 ? mask : nullptr;
  a.mbool = mask_kind == TA_MASK_BOOL ? static_cast<const uint32_t *>(mask) : nullptr;
  a.out = out;
  a.mask_head_stride = mask ? mask_head_stride : 0;
  a.mask_stride = mask ? mask_stride : kv_seq_len;
  a.batch = batch;
  a.nq = n_q_heads;
  a.nkv = n_kv_heads;
  a.repeat = n_q_heads / n_kv_heads;
  a.kv_seq_len = kv_seq_len;
  a.kv_capacity = kv_capacity;
  a.q_l = q_l;
  a.nwg = nwg;
  a.rows = (uint32_t)rows;
  a.row_tiles = ceil_div(a.rows, ta::kQuantRowsPerWG);
  a.n_tiles = ceil_div(kv_seq_len, ta::quant_tile_keys(dim));
  // window: the last window_size tokens ("ffai/flash_quantized_sdpa.rs",
  // token t is kept iff t + window_size > kv_seq_len - 1); 0 or a window
  // at least as long as the sequence keeps every token
  a.key_lo = (window_size > 0 && window_size < kv_seq_len) ? kv_seq_len - window_size : 0;
  uint64_t units = BnKV * nwg;
  uint64_t blocks = (uint64_t)ta::kXcds * ((units + ta::kXcds - 1) / ta::kXcds) * a.row_tiles;
  if (blocks > 0x7fffffffull)
    return fail(TA_EUNSUPPORTED, "%s: grid too large", fn);
  a.units = (uint32_t)units;
  a.qscale = scale * ta::kLog2e;
  if (nwg > 1) {
    a.part_o = partials;
    a.part_sm = partials + (size_t)nwg * BnQ * q_l * dim;
  } else {
    a.part_o = a.part_sm = nullptr;
  }
  return hip_status(ta::launch_quant_forward(a, dim, bits, group_size,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

int tree_attn_quant_forward(
    const void *q, int q_dtype, size_t q_bytes, const uint32_t *k_packed,
    const void *k_scales, const void *k_biases, const uint32_t *v_packed,
    const void *v_scales, const void *v_biases, const size_t kv_bytes[6],
    const float *sinks, size_t sinks_bytes, const void *mask,
    size_t mask_bytes, uint64_t mask_head_stride, uint32_t mask_stride,
    float *partials, size_t partials_bytes, void *out, size_t out_bytes,
    uint32_t batch, uint32_t n_q_heads, uint32_t n_kv_heads, uint32_t dim,
    uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l, uint32_t bits,
    uint32_t group_size, float scale, uint32_t nwg, void *stream) {
  return quant_forward("tree_attn_quant_forward", q, q_dtype, q_bytes, k_packed, k_scales,
                       k_biases, v_packed, v_scales, v_biases, kv_bytes, sinks, sinks_bytes,
                       mask, mask ? TA_MASK_F16 : TA_MASK_NONE, mask_bytes, mask_head_stride,
                       mask_stride, 0u, partials, partials_bytes, out, out_bytes, batch,
                       n_q_heads, n_kv_heads, dim, kv_seq_len, kv_capacity, q_l, bits,
                       group_size, scale, nwg, stream);
}

int tree_attn_quant_forward_ex(
    const void *q, int q_dtype, size_t q_bytes, const uint32_t *k_packed,
    const void *k_scales, const void *k_biases, const uint32_t *v_packed,
    const void *v_scales, const void *v_biases, const size_t kv_bytes[6],
    const float *sinks, size_t sinks_bytes, const void *mask, int mask_kind,
    size_t mask_bytes, uint64_t mask_head_stride, uint32_t mask_stride,
    uint32_t window_size, float *partials, size_t partials_bytes, void *out,
    size_t out_bytes, uint32_t batch, uint32_t n_q_heads, uint32_t n_kv_heads,
    uint32_t dim, uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
    uint32_t bits, uint32_t group_size, float scale, uint32_t nwg, void *stream) {
  return quant_forward("tree_attn_quant_forward_ex", q, q_dtype, q_bytes, k_packed,
                       k_scales, k_biases, v_packed, v_scales, v_biases, kv_bytes, sinks,
                       sinks_bytes, mask, mask_kind, mask_bytes, mask_head_stride, mask_stride,
                       window_size, partials, partials_bytes, out, out_bytes, batch, n_q_heads,
                       n_kv_heads, dim, kv_seq_len, kv_capacity, q_l, bits, group_size, scale,
                       nwg, stream);
}

int build_tree_mask(const int32_t *parents, uint32_t q_l, uint32_t kv_seq_len,
                    uint32_t mask_stride, float *mask, size_t mask_bytes,
                    void *stream) {
  const char *fn = "build_tree_mask";
  if (q_l == 0) return fail(TA_EINVAL, "%s: q_l must be > 0", fn);
  if (q_l > (uint32_t)ta::kMaxTreeNodes)
    return fail(TA_EUNSUPPORTED, "%s: q_l must be <= %d, got %u", fn, ta::kMaxTreeNodes, q_l);
  if (kv_seq_len < q_l)
    return fail(TA_EINVAL, "%s: kv_seq_len %u is shorter than the q_l %u tree nodes", fn, kv_seq_len, q_l);
  if (mask_stride < kv_seq_len)
    return fail(TA_EINVAL, "%s: mask_stride %u is shorter than kv_seq_len %u", fn, mask_stride,
                kv_seq_len);
  if (!parents || !mask) return fail(TA_EINVAL, "%s: parents and mask must not be NULL", fn);
  if ((uintptr_t)mask & 3u) return fail(TA_EINVAL, "%s: mask must be 4-byte aligned", fn);
  if (parents[0] != -1)
    return fail(TA_EINVAL, "%s: invalid topology: parents[0] must be -1, got %d", fn,
                parents[0]);
  for (uint32_t i = 1; i < q_l; ++i)
    if (parents[i] < 0 || (uint32_t)parents[i] >= i)
      return fail(TA_EINVAL, "%s: invalid topology: parents[%u] = %d (need 0 <= p < %u)", fn,
                  i, parents[i], i);
  uint64_t req;
  if (!mul3(q_l, mask_stride, 4, req)) return fail(TA_EOVERFLOW, "%s: size overflows", fn);
  if (mask_bytes < req)
    return fail(TA_ESIZE, "%s: mask buffer holds %zu bytes of the %llu needed", fn,
                mask_bytes, (unsigned long long)req);
  ta::MaskArgs a;
  memset(a.parents, 0, sizeof a.parents);
  for (uint32_t i = 0; i < q_l; ++i) a.parents[i] = (int16_t)parents[i];
  a.mask = mask;
  a.q_l = q_l;
  a.kv_seq_len = kv_seq_len;
  a.mask_stride = mask_stride;
  return hip_status(ta::launch_tree_mask(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
