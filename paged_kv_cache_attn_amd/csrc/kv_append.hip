// kv_append: store new tokens' key/value vectors in the paged cache.
//
// A growing sequence writes its new tokens into the blocks it owns (possibly
// freshly allocated ones) and nothing already stored moves ("Ultimate Guide
// to PagedAttention", newline: KV cache and dynamic growth).  Token t goes to
// slot s = slot_mapping[t]: block s >> log2(bs), offset s & (bs - 1); K is a
// token-major row of the (block, kv-head) slab, V a column of its 16-token
// dimension-major sub-slab.  The copy is of raw bits.  Also the whole-block
// copy that copy-on-write needs.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

// One work-group per (run of 16 consecutive new tokens, kv-head).  K rows
// are copied with 16-byte pieces.  When the run's slots are the 16 columns of
// one V sub-slab, in order (a prefill chunk appended to its own blocks), the
// run's V is transposed through LDS and the whole [D x 16] sub-slab is
// written with 16-byte stores; otherwise each token's V column is written
// element by element.
template <typename W>  // W: uint16_t (bf16) or uint32_t (fp32) -- a raw element
__global__ __launch_bounds__(256) void kv_append_kernel(const AppendArgs a) {
  constexpr int kRun = 16;
  constexpr int EPP = 16 / (int)sizeof(W);  // elements per 16-byte piece
  constexpr int kPer = 2;                   // pieces per thread: 16 rows x D / EPP <= 512
  __shared__ int slot_s[kRun];
  __shared__ __attribute__((aligned(16))) W vt[kRun * 128];  // [token][d], D <= 128
  const int h = blockIdx.x % a.Hkv;
  const int t0 = (blockIdx.x / a.Hkv) * kRun;
  const int ntok = min(kRun, a.T - t0);
  const int tid = threadIdx.x;
  const int D = a.D;
  const int bs = 1 << a.bs_log2;
  const int ppr = D / EPP;  // pieces per row
  const W* kn = static_cast<const W*>(a.k_new);
  const W* vn = static_cast<const W*>(a.v_new);
  W* kc = static_cast<W*>(a.k_cache);
  W* vc = static_cast<W*>(a.v_cache);
  // The new rows' K and V pieces are loaded first: their addresses do not
  // depend on the slots, so these loads overlap the slot-mapping read.
  u32x4 kx[kPer], vx[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = tid + 256 * j;
    const int i = p / ppr, c = p - i * ppr;
    if (p < kRun * ppr && i < ntok) {
      const size_t src = ((size_t)(t0 + i) * a.Hkv + h) * D + c * EPP;
      kx[j] = *reinterpret_cast<const u32x4*>(kn + src);
      vx[j] = *reinterpret_cast<const u32x4*>(vn + src);
    }
  }
  if (tid < kRun) slot_s[tid] = tid < ntok ? a.slots[t0 + tid] : -1;
  __syncthreads();
  const int s0 = slot_s[0];
  bool whole = ntok == kRun && s0 >= 0 && (s0 & (kRun - 1)) == 0;
#pragma unroll
  for (int i = 1; i < kRun; ++i) whole = whole && slot_s[i] == s0 + i;

  const size_t slab = (size_t)bs * D;  // elements of one (block, kv-head) slab
  // K: 16-byte pieces of each token's row
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = tid + 256 * j;
    const int i = p / ppr, c = p - i * ppr;
    if (p >= kRun * ppr || i >= ntok) continue;
    const int slot = slot_s[i];
    if (slot < 0) continue;
    PA_DEVICE_CHECK((slot >> a.bs_log2) < a.num_blocks);
    const int blk = slot >> a.bs_log2, off = slot & (bs - 1);
    *reinterpret_cast<u32x4*>(kc + ((size_t)blk * a.Hkv + h) * slab + (size_t)off * D + c * EPP) = kx[j];
  }
  if (whole) {
    // V rows of the run into LDS, then the sub-slab [D][16] with 16-byte stores
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = tid + 256 * j;
      const int i = p / ppr, c = p - i * ppr;
      if (p < kRun * ppr) *reinterpret_cast<u32x4*>(&vt[i * D + c * EPP]) = vx[j];
    }
    __syncthreads();
    const int blk = s0 >> a.bs_log2, off = s0 & (bs - 1);
    PA_DEVICE_CHECK(blk < a.num_blocks);
    W* sub = vc + ((size_t)blk * a.Hkv + h) * slab + (size_t)(off >> 4) * D * kRun;
    constexpr int PPD = kRun / EPP;  // pieces per sub-slab row
    for (int p = tid; p < D * PPD; p += 256) {
      const int d = p / PPD, c = p - d * PPD;
      W e[EPP];
#pragma unroll
      for (int k = 0; k < EPP; ++k) e[k] = vt[(c * EPP + k) * D + d];
      *reinterpret_cast<u32x4*>(sub + (size_t)d * kRun + c * EPP) = __builtin_bit_cast(u32x4, e);
    }
  } else {
    // scattered slots: a 16-byte piece of a token's V row per thread, written
    // element by element down the token's sub-slab column
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = tid + 256 * j;
      const int i = p / ppr, c = p - i * ppr;
      if (p >= kRun * ppr || i >= ntok) continue;
      const int slot = slot_s[i];
      if (slot < 0) continue;
      PA_DEVICE_CHECK((slot >> a.bs_log2) < a.num_blocks);
      const int blk = slot >> a.bs_log2, off = slot & (bs - 1);
      W e[EPP];
      __builtin_memcpy(e, &vx[j], 16);
      W* col = vc + ((size_t)blk * a.Hkv + h) * slab + (size_t)(off >> 4) * D * kRun + (off & 15);
#pragma unroll
      for (int k = 0; k < EPP; ++k) col[(size_t)(c * EPP + k) * kRun] = e[k];
    }
  }
}

// Copy-on-write: whole (block, kv-head) slabs of K and V, bit for bit.  One
// work-group per (pair, kv-head, K or V); 16-byte loads and stores.
__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyArgs a) {
  const int which = blockIdx.x & 1;  // 0: K, 1: V
  const int rest = blockIdx.x >> 1;
  const int h = rest % a.Hkv;
  const int i = rest / a.Hkv;
  const size_t slab = (size_t)a.slab16;
  PA_DEVICE_CHECK(a.src[i] >= 0 && a.src[i] < a.num_blocks && a.dst[i] >= 0 && a.dst[i] < a.num_blocks);
  const size_t src = ((size_t)a.src[i] * a.Hkv + h) * slab;
  const size_t dst = ((size_t)a.dst[i] * a.Hkv + h) * slab;
  u32x4* pool = static_cast<u32x4*>(which ? a.v_cache : a.k_cache);
  for (size_t u = threadIdx.x; u < slab; u += 256) pool[dst + u] = pool[src + u];
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.pairs * a.Hkv * 2;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int dtype, hipStream_t s) {
  const long long blocks = ((long long)a.T + 15) / 16 * a.Hkv;
  if (blocks <= 0) return hipSuccess;
  if (dtype == 1) {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
