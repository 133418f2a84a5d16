// C ABI of the exact-attention library: argument validation, dispatch to the
// gfx950 kernels, status strings.  Every check runs on the host before any
// HIP call, so invalid arguments never launch anything and never touch the
// outputs.
#include "fa.h"
#include "fa_internal.hpp"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <atomic>
#include <mutex>

// Scratch memory of fa_backward_noalloc: the backward workspace (the two
// float32 row vectors D and LSE * log2(e)) for callers that cannot allocate
// device memory.  Every GPU the library runs on holds its own copy until the
// process ends.  Host code never uses this name as an address: the address
// on a device comes from hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

int check_sizes(int B, int H, int n_q, int n_k, int d, int dtype) {
  if (B < 1 || H < 1 || n_q < 1 || n_k < 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * (long long)H > INT_MAX) return FA_ERR_INVALID_ARG;
  // Workgroups per launch: at most ceil(n / 32) per (batch, head).
  const long long tiles = ((long long)(n_q > n_k ? n_q : n_k) + 31) / 32;
  if (tiles * (long long)B * (long long)H > INT_MAX) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Finite test on the bit pattern: the library is built without NaN semantics
// (-fno-honor-nans), under which std::isfinite may be folded to true.
bool finite_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof(u));
  return ((u >> 23) & 0xFFu) != 0xFFu;
}

int check_scale_causal(float scale, int causal) {
  if (!finite_bits(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int check_tensor(const void* p) {
  if (p == nullptr) return FA_ERR_INVALID_ARG;
  if (!aligned(p, 16)) return FA_ERR_ALIGNMENT;
  return FA_OK;
}

int check_rowvec(const float* p) {
  if (p == nullptr) return FA_ERR_INVALID_ARG;
  if (!aligned(p, 4)) return FA_ERR_ALIGNMENT;
  return FA_OK;
}

// First nonzero status of a list of checks.
template <typename... T>
int first_error(T... s) {
  int r = FA_OK;
  ((r = (r != FA_OK ? r : s)), ...);
  return r;
}

// Backward workspace: two float32 (B,H,n_q) row vectors, D then LSE*log2(e),
// each followed by at least 16 bytes of slack (16-byte copies of a vector's
// last entries may read up to 12 bytes past it) and rounded up to 256 bytes.
size_t ws_half_bytes(int B, int H, int n_q) {
  const size_t raw = (size_t)B * (size_t)H * (size_t)n_q * sizeof(float) + 16;
  return (raw + 255) / 256 * 256;
}
size_t ws_bytes(int B, int H, int n_q) { return 2 * ws_half_bytes(B, H, n_q); }

int check_workspace(const void* ws, size_t bytes, int B, int H, int n_q) {
  if (ws == nullptr || bytes < ws_bytes(B, H, n_q)) return FA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return FA_ERR_ALIGNMENT;
  return FA_OK;
}

// Shared K/V heads in the backward pass: a K/V head's query heads are split
// into `slices` runs (a divisor of the group size), each dK/dV workgroup
// taking one run, and each run leaves float32 partial dK and dV after the two
// row vectors of the workspace.  Runs of one query head give the most
// parallel work and keep the dK/dV kernel free of a head loop (which costs it
// 72 spilled registers); the runs grow only when the partials would pass
// kBwdPartLimit bytes.
// Keys per dK/dV workgroup at the narrowest routing: the bf16 kernel takes
// 64 keys (two waves) on causal, windowed and nearly empty passes and 128
// otherwise, the fp32 kernel 128; the grid-size guard counts 64-key tiles,
// the most workgroups any routing launches.
constexpr int kBwdKeyTile = 64;
constexpr double kBwdPartLimit = 4294967296.0;
int bwd_slices(int B, int H, int H_kv, int n_k) {
  const int group = H / H_kv;
  for (int sl = group; sl > 1; --sl)
    if (group % sl == 0 && 2.0 * sl * B * H_kv * n_k * 128 * 4 <= kBwdPartLimit) return sl;
  return 1;
}
size_t part_bytes(int B, int H_kv, int n_k, int d, int slices) {
  return slices > 1 ? round256((size_t)slices * B * H_kv * n_k * d * sizeof(float)) : 0;
}
size_t gqa_ws_bytes(int B, int H, int H_kv, int n_q, int n_k, int d) {
  return ws_bytes(B, H, n_q) + 2 * part_bytes(B, H_kv, n_k, d, bwd_slices(B, H, H_kv, n_k));
}

fa::BwdArgs make_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, const void* ws, void* dq, void* dk, void* dv, int B, int H,
                     int n_q, int n_k, float scale, int H_kv, int q_offset = 0, int window = -1) {
  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
  char* w = static_cast<char*>(const_cast<void*>(ws));
  a.delta = reinterpret_cast<float*>(w);
  a.lse2 = w ? reinterpret_cast<float*>(w + ws_half_bytes(B, H, n_q)) : nullptr;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.BH = B * H; a.H = H; a.group = H / H_kv; a.n_q = n_q; a.n_k = n_k;
  a.q_offset = q_offset; a.window = window;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.slices = 1;
  a.part_dk = a.part_dv = nullptr;
  return a;
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

fa::FwdArgs make_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int H_kv, int n_q, int n_k, float scale, int q_offset, int window) {
  fa::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = B * H; a.H = H; a.group = H / H_kv; a.n_q = n_q; a.n_k = n_k;
  a.q_offset = q_offset; a.window = window;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_prior = nullptr;
  a.lse_prior = nullptr;
  a.prior_f32 = 0;
  a.out_f32 = 0;
  return a;
}

// Split-KV decoding.  Chunks hold whole key blocks and at least
// kDecodeMinChunk keys; the default aims at kDecodeTargetWgs workgroups (one
// per compute unit).
constexpr int kDecodeMinChunk = 256;
constexpr long long kDecodeTargetWgs = 256;
constexpr int kDecodeMaxSplits = 65536;

// Workspace: float32 partial outputs (n_splits, B*H*n_q, d), then partial
// LSE (n_splits, B*H*n_q), each rounded up to 256 bytes.
size_t dec_part_o_bytes(int B, int H, int n_q, int d, int n_splits) {
  return round256((size_t)n_splits * B * H * n_q * d * sizeof(float));
}
size_t dec_ws_bytes(int B, int H, int n_q, int d, int n_splits) {
  if (n_splits <= 1) return 0;
  return dec_part_o_bytes(B, H, n_q, d, n_splits) + round256((size_t)n_splits * B * H * n_q * sizeof(float));
}

// H_kv K/V heads shared by groups of H / H_kv consecutive query heads.
int check_kv_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Query offset and window half-width within +-2^29, and with either of them
// in use also n_q, n_k <= 2^29, so that the position arithmetic of the mask
// (row + offset +- window) stays within 32-bit ints; window -1 means none.
constexpr int kMaxBand = 1 << 29;
int check_band(int n_q, int n_k, int q_offset, int window) {
  if (q_offset < -kMaxBand || q_offset > kMaxBand) return FA_ERR_INVALID_ARG;
  if (window < -1 || window > kMaxBand) return FA_ERR_INVALID_ARG;
  if ((q_offset != 0 || window != -1) && (n_q > kMaxBand || n_k > kMaxBand))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// The decode kernel's launch for validated arguments: n_splits chunks of the
// key axis (workspace as dec_ws_bytes when more than one holds keys).
int decode_launch(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                  size_t workspace_bytes, int B, int H, int H_kv, int n_q, int n_k, int d,
                  float scale, int causal, int q_offset, int window, int n_splits, void* stream) {
  const long long rows = (long long)(H / H_kv) * n_q;
  const long long n_rb = (rows + 31) / 32;
  long long chunk = ((long long)n_k + n_splits - 1) / n_splits;
  chunk = (chunk + fa::kDecodeBlock - 1) / fa::kDecodeBlock * fa::kDecodeBlock;
  const long long splits = ((long long)n_k + chunk - 1) / chunk;  // chunks that hold keys
  if (rows > INT_MAX || (long long)B * H_kv * splits * n_rb > INT_MAX) return FA_ERR_INVALID_ARG;
  if (splits > 1) {
    if (workspace == nullptr || workspace_bytes < dec_ws_bytes(B, H, n_q, d, n_splits)) return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGNMENT;
  }
  fa::DecArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  char* w = static_cast<char*>(workspace);
  a.part_o = splits > 1 ? reinterpret_cast<float*>(w) : nullptr;
  a.part_lse = splits > 1 ? reinterpret_cast<float*>(w + dec_part_o_bytes(B, H, n_q, d, n_splits)) : nullptr;
  a.B = B; a.H = H; a.group = H / H_kv; a.h_kv = H_kv;
  a.n_q = n_q; a.n_k = n_k; a.q_offset = q_offset; a.window = window;
  a.rows = (int)rows; a.n_rb = (int)n_rb;
  a.n_splits = (int)splits; a.chunk = (int)chunk;
  a.scale_log2 = scale * 1.4426950408889634f;
  return status_of(fa::launch_decode_bf16(a, d, causal != 0, static_cast<hipStream_t>(stream)));
}

// Shapes too small in B*H*n_q to fill the GPU with the forward kernel's
// 256-row workgroups (one wave of a workgroup walks every key for its 32
// rows) but with many keys: the decode kernel with one chunk spreads the keys
// of each 32-row block over four waves and merges them in LDS, without a
// workspace.  Measured on MI355X (bf16, one chunk vs forward): 1.6-2.1x
// faster at up to 32 such tiles for d = 32, 64, 128 (n_k >= 1024); at 64
// tiles 1.35-1.75x for d <= 64 but 0.92x for d = 128.
constexpr long long kStarvedTiles = 32;
constexpr long long kStarvedTilesNarrow = 64;  // d <= 64
constexpr int kStarvedMinKeys = 1024;
bool starved(int B, int H, int n_q, int n_k, int d) {
  const long long tiles = (long long)B * H * ((n_q + 255) / 256);
  return n_k >= kStarvedMinKeys && tiles <= (d <= 64 ? kStarvedTilesNarrow : kStarvedTiles);
}

// Float32 shapes that leave compute units idle with the forward kernel's
// 128-row workgroups: the key-split kernel runs one 32-row block per
// workgroup, its keys spread over four waves.  It does about 15 % less work
// per compute unit, so it pays while it reaches at least twice as many
// (measured on MI355X up to 128 tiles, from 128 keys up: c1 10.5 -> 6.7 us,
// c2 341 -> 101 us; B=1 H=32 n=512 d=64 causal 50.2 -> 35.7 us).
constexpr long long kStarvedTilesF32 = 128;
bool starved_f32(int B, int H, int n_q) {
  const long long tiles = (long long)B * H * ((n_q + 127) / 128);
  return tiles <= kStarvedTilesF32;
}
// Among those, shapes whose 32-row blocks would fill at most half of the 256
// compute units take 16-row blocks (16x16x4 products: twice the LDS reads per
// product, so only where the blocks are that few).  Measured on MI355X: c2
// 100.2 -> 78.1 us, d = 128 194.5 -> 147.0 us, B=1 H=4 1024 x 8192 keys
// d = 128 377.3 -> 285.8 us; at 256 blocks of 32 (H=2, n=4096, d=64)
// 102.0 -> 114.1 us, where 32-row blocks stay.
constexpr long long kStarvedBlocks16 = 128;
bool starved_f32_16(int B, int H, int n_q) {
  return (long long)B * H * ((n_q + 31) / 32) <= kStarvedBlocks16;
}

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int H_kv, int n_q, int n_k, int d, float scale, int causal, int dtype,
                 void* stream, int q_offset = 0, int window = -1) {
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_kv_heads(H, H_kv),
                       check_band(n_q, n_k, q_offset, window), check_scale_causal(scale, causal),
                       check_tensor(q), check_tensor(k), check_tensor(v), check_tensor(o),
                       check_rowvec(lse));
  if (st != FA_OK) return st;
  if (dtype == FA_DTYPE_BF16 && starved(B, H, n_q, n_k, d))
    return decode_launch(q, k, v, o, lse, nullptr, 0, B, H, H_kv, n_q, n_k, d, scale, causal,
                         q_offset, window, 1, stream);
  fa::FwdArgs a = make_fwd(q, k, v, o, lse, B, H, H_kv, n_q, n_k, scale, q_offset, window);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_DTYPE_FP32 && starved_f32(B, H, n_q))
    return status_of(starved_f32_16(B, H, n_q) ? fa::launch_fwd_f32_split16(a, d, causal != 0, s)
                                               : fa::launch_fwd_f32_split(a, d, causal != 0, s));
  return status_of(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, d, causal != 0, s)
                                          : fa::launch_fwd_f32(a, d, causal != 0, s));
}

// Byte ranges [p, p + n) and [r, r + m) overlap.
bool overlap(const void* p, size_t n, const void* r, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(r);
  return a < b + m && b < a + n;
}

int forward_merge_impl(const void* q, const void* k, const void* v, const void* o_prior,
                       const float* lse_prior, int prior_dtype, void* o, float* lse, int out_dtype,
                       int B, int H, int H_kv, int n_q, int n_k, int d, float scale, int causal,
                       int q_offset, int window, int dtype, void* stream) {
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_kv_heads(H, H_kv),
                       check_band(n_q, n_k, q_offset, window), check_scale_causal(scale, causal),
                       check_tensor(q), check_tensor(k), check_tensor(v), check_tensor(o_prior),
                       check_rowvec(lse_prior), check_tensor(o), check_rowvec(lse));
  if (st != FA_OK) return st;
  // The running result is float32 or the input dtype (float32 inputs: float32 only).
  const auto acc_ok = [dtype](int t) { return t == FA_DTYPE_FP32 || t == dtype; };
  if (!acc_ok(prior_dtype) || !acc_ok(out_dtype)) return FA_ERR_UNSUPPORTED;
  // o may be o_prior itself (same dtype) and lse may be lse_prior; any other
  // overlap between them is refused.
  const size_t rows = (size_t)B * H * n_q;
  const size_t pb = rows * d * (prior_dtype == FA_DTYPE_FP32 ? 4 : 2);
  const size_t ob = rows * d * (out_dtype == FA_DTYPE_FP32 ? 4 : 2);
  if (o == o_prior ? prior_dtype != out_dtype : overlap(o, ob, o_prior, pb)) return FA_ERR_INVALID_ARG;
  if (lse != lse_prior && overlap(lse, rows * 4, lse_prior, rows * 4)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a = make_fwd(q, k, v, o, lse, B, H, H_kv, n_q, n_k, scale, q_offset, window);
  a.o_prior = o_prior;
  a.lse_prior = lse_prior;
  a.prior_f32 = prior_dtype == FA_DTYPE_FP32;
  a.out_f32 = out_dtype == FA_DTYPE_FP32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_merge_bf16(a, d, causal != 0, s)
                                          : fa::launch_fwd_merge_f32(a, d, causal != 0, s));
}

int backward_impl(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, int B, int H, int H_kv, int n_q, int n_k, int d,
                  float scale, int causal, int dtype, void* stream, int q_offset = 0,
                  int window = -1) {
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_kv_heads(H, H_kv),
                       check_band(n_q, n_k, q_offset, window),
                       check_scale_causal(scale, causal), check_tensor(q), check_tensor(k),
                       check_tensor(v), check_tensor(o), check_tensor(dO), check_rowvec(lse),
                       check_tensor(dq), check_tensor(dk), check_tensor(dv));
  if (st != FA_OK) return st;
  st = check_workspace(workspace, workspace_bytes, B, H, n_q);
  if (st != FA_OK) return st;
  const int slices = bwd_slices(B, H, H_kv, n_k);
  if (workspace_bytes < gqa_ws_bytes(B, H, H_kv, n_q, n_k, d)) return FA_ERR_WORKSPACE;
  if ((long long)((n_k + kBwdKeyTile - 1) / kBwdKeyTile) * B * H_kv * slices > INT_MAX)
    return FA_ERR_INVALID_ARG;
  fa::BwdArgs a = make_bwd(q, k, v, o, dO, lse, workspace, dq, dk, dv, B, H, n_q, n_k, scale, H_kv,
                           q_offset, window);
  a.slices = slices;
  if (slices > 1) {
    char* w = static_cast<char*>(workspace) + ws_bytes(B, H, n_q);
    a.part_dk = reinterpret_cast<float*>(w);
    a.part_dv = reinterpret_cast<float*>(w + part_bytes(B, H_kv, n_k, d, slices));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == FA_DTYPE_BF16;
  hipError_t e = fa::launch_bwd_preprocess(a, d, bf16, s);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  e = bf16 ? fa::launch_bwd_dkdv_bf16(a, d, causal != 0, s)
           : fa::launch_bwd_dkdv_f32(a, d, causal != 0, s);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  if (slices > 1) {
    e = fa::launch_bwd_reduce_slices(a, d, bf16, s);
    if (e != hipSuccess) return FA_ERR_LAUNCH;
  }
  e = bf16 ? fa::launch_bwd_dq_bf16(a, d, causal != 0, s)
           : fa::launch_bwd_dq_f32(a, d, causal != 0, s);
  return status_of(e);
}

// The device address of `scratch` on the device of `stream` (which must be
// the calling thread's current device), looked up once per device with that
// device current and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void* stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
  if (stream != nullptr) {
    hipDevice_t dev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess || dev != cur)
      return FA_ERR_INVALID_ARG;
  }
  if (cur < 0 || cur >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[cur] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_LAUNCH;
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return FA_OK;
}

}  // namespace

namespace fa {

int compute_units(hipStream_t stream) {
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return 0;
    dev = d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return 0;
  }
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fa

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head width or dtype";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ALIGNMENT: return "tensor pointer misaligned";
    case FA_ERR_TOO_LARGE: return "sizes exceed the fixed scratch of the non-allocating entry point";
    default: return "unknown status";
  }
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int n_q, int n_k, int d, float scale, int causal, int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, H, n_q, n_k, d, scale, causal, dtype, stream);
}

int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int H_kv, int n_q, int n_k, int d, float scale, int causal, int dtype,
                   void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, H_kv, n_q, n_k, d, scale, causal, dtype, stream);
}

size_t fa_backward_workspace_size(int B, int H, int n_q, int n_k, int d, int dtype) {
  if (check_sizes(B, H, n_q, n_k, d, dtype) != FA_OK) return 0;
  return ws_bytes(B, H, n_q);
}

size_t fa_backward_gqa_workspace_size(int B, int H, int H_kv, int n_q, int n_k, int d, int dtype) {
  if (check_sizes(B, H, n_q, n_k, d, dtype) != FA_OK || check_kv_heads(H, H_kv) != FA_OK) return 0;
  return gqa_ws_bytes(B, H, H_kv, n_q, n_k, d);
}

int fa_backward_preprocess(const void* o, const void* dO, const float* lse, void* workspace,
                           size_t workspace_bytes, int B, int H, int n_q, int d, int dtype,
                           void* stream) {
  int st = first_error(check_sizes(B, H, n_q, 1, d, dtype), check_tensor(o), check_tensor(dO),
                       check_rowvec(lse), check_workspace(workspace, workspace_bytes, B, H, n_q));
  if (st != FA_OK) return st;
  fa::BwdArgs a = make_bwd(nullptr, nullptr, nullptr, o, dO, lse, workspace, nullptr, nullptr,
                           nullptr, B, H, n_q, 1, 0.f, H);
  return status_of(fa::launch_bwd_preprocess(a, d, dtype == FA_DTYPE_BF16,
                                             static_cast<hipStream_t>(stream)));
}

int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO,
                     const void* workspace, size_t workspace_bytes, void* dk, void* dv, int B,
                     int H, int n_q, int n_k, int d, float scale, int causal, int dtype,
                     void* stream) {
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_scale_causal(scale, causal),
                       check_tensor(q), check_tensor(k), check_tensor(v), check_tensor(dO),
                       check_workspace(workspace, workspace_bytes, B, H, n_q), check_tensor(dk),
                       check_tensor(dv));
  if (st != FA_OK) return st;
  fa::BwdArgs a = make_bwd(q, k, v, nullptr, dO, nullptr, workspace, nullptr, dk, dv, B, H, n_q,
                           n_k, scale, H);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == FA_DTYPE_BF16 ? fa::launch_bwd_dkdv_bf16(a, d, causal != 0, s)
                                          : fa::launch_bwd_dkdv_f32(a, d, causal != 0, s));
}

int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO,
                   const void* workspace, size_t workspace_bytes, void* dq, int B, int H, int n_q,
                   int n_k, int d, float scale, int causal, int dtype, void* stream) {
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_scale_causal(scale, causal),
                       check_tensor(q), check_tensor(k), check_tensor(v), check_tensor(dO),
                       check_workspace(workspace, workspace_bytes, B, H, n_q), check_tensor(dq));
  if (st != FA_OK) return st;
  fa::BwdArgs a = make_bwd(q, k, v, nullptr, dO, nullptr, workspace, dq, nullptr, nullptr, B, H,
                           n_q, n_k, scale, H);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == FA_DTYPE_BF16 ? fa::launch_bwd_dq_bf16(a, d, causal != 0, s)
                                          : fa::launch_bwd_dq_f32(a, d, causal != 0, s));
}

int fa_forward_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int H_kv, int n_q, int n_k, int d, float scale, int causal, int q_offset,
                   int window, int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, H_kv, n_q, n_k, d, scale, causal, dtype, stream,
                      q_offset, window);
}

int fa_forward_merge(const void* q, const void* k, const void* v, const void* o_prior,
                     const float* lse_prior, int prior_dtype, void* o, float* lse, int out_dtype,
                     int B, int H, int H_kv, int n_q, int n_k, int d, float scale, int causal,
                     int q_offset, int window, int dtype, void* stream) {
  return forward_merge_impl(q, k, v, o_prior, lse_prior, prior_dtype, o, lse, out_dtype, B, H, H_kv,
                            n_q, n_k, d, scale, causal, q_offset, window, dtype, stream);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int H, int n_q, int n_k, int d, float scale,
                int causal, int dtype, void* stream) {
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, n_q,
                       n_k, d, scale, causal, dtype, stream);
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int n_q, int n_k,
                        int d, float scale, int causal, int dtype, void* stream) {
  // Everything that can be checked without the GPU first, the scratch size
  // included; the scratch is only looked up for a call that will launch.
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_scale_causal(scale, causal),
                       check_tensor(q), check_tensor(k), check_tensor(v), check_tensor(o),
                       check_tensor(dO), check_rowvec(lse), check_tensor(dq), check_tensor(dk),
                       check_tensor(dv));
  if (st != FA_OK) return st;
  if (ws_bytes(B, H, n_q) > kNoAllocScratchBytes) return FA_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = noalloc_scratch(stream, &ws);
  if (st != FA_OK) return st;
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, ws, kNoAllocScratchBytes, B, H, H, n_q, n_k,
                       d, scale, causal, dtype, stream);
}

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, int B, int H, int H_kv, int n_q, int n_k, int d,
                    float scale, int causal, int dtype, void* stream) {
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H_kv,
                       n_q, n_k, d, scale, causal, dtype, stream);
}

int fa_backward_ext(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, int B, int H, int H_kv, int n_q, int n_k, int d,
                    float scale, int causal, int q_offset, int window, int dtype, void* stream) {
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H_kv,
                       n_q, n_k, d, scale, causal, dtype, stream, q_offset, window);
}


int fa_lse_merge(const void* o_parts, const float* lse_parts, void* o, float* lse, int n_parts,
                 long long rows, int d, int parts_dtype, int out_dtype, void* stream) {
  if (n_parts < 1 || rows < 1) return FA_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const auto dtype_ok = [](int t) { return t == FA_DTYPE_FP32 || t == FA_DTYPE_BF16; };
  if (!dtype_ok(parts_dtype) || !dtype_ok(out_dtype)) return FA_ERR_UNSUPPORTED;
  int st = first_error(check_tensor(o_parts), check_tensor(o), check_rowvec(lse_parts), check_rowvec(lse));
  if (st != FA_OK) return st;
  const long long rows_per_wg = 256 / (d / 4);
  if ((rows + rows_per_wg - 1) / rows_per_wg > INT_MAX) return FA_ERR_INVALID_ARG;
  if ((double)n_parts * (double)rows * d > 9.0e15) return FA_ERR_INVALID_ARG;
  fa::MergeArgs m;
  m.o_parts = o_parts;
  m.lse_parts = lse_parts;
  m.o = o;
  m.lse = lse;
  m.rows = rows;
  m.n_parts = n_parts;
  return status_of(fa::launch_lse_merge(m, d, parts_dtype == FA_DTYPE_BF16, out_dtype == FA_DTYPE_BF16,
                                        static_cast<hipStream_t>(stream)));
}

size_t fa_decode_workspace_size(int B, int H, int n_q, int d, int n_splits) {
  if (B < 1 || H < 1 || n_q < 1 || n_splits < 1 || n_splits > kDecodeMaxSplits) return 0;
  if (d != 32 && d != 64 && d != 128) return 0;
  return dec_ws_bytes(B, H, n_q, d, n_splits);
}

int fa_decode_splits(int B, int H, int H_kv, int n_q, int n_k) {
  if (B < 1 || H < 1 || n_q < 1 || n_k < 1 || check_kv_heads(H, H_kv) != FA_OK) return 0;
  const long long rows = (long long)(H / H_kv) * n_q;
  const long long units = (long long)B * H_kv * ((rows + 31) / 32);
  const long long most = std::max(1LL, (long long)n_k / kDecodeMinChunk);
  const long long want = (kDecodeTargetWgs + units - 1) / units;
  return (int)std::max(1LL, std::min(want, most));
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
              size_t workspace_bytes, int B, int H, int H_kv, int n_q, int n_k, int d, float scale,
              int causal, int q_offset, int window, int n_splits, int dtype, void* stream) {
  int st = first_error(check_sizes(B, H, n_q, n_k, d, dtype), check_kv_heads(H, H_kv),
                       check_band(n_q, n_k, q_offset, window), check_scale_causal(scale, causal),
                       check_tensor(q), check_tensor(k), check_tensor(v), check_tensor(o),
                       check_rowvec(lse));
  if (st != FA_OK) return st;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (n_splits < 1 || n_splits > kDecodeMaxSplits) return FA_ERR_INVALID_ARG;
  return decode_launch(q, k, v, o, lse, workspace, workspace_bytes, B, H, H_kv, n_q, n_k, d, scale,
                       causal, q_offset, window, n_splits, stream);
}

}  // extern "C"
