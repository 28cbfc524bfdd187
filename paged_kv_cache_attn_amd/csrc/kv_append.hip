// kv_append: store new tokens' key/value vectors in the paged cache.
//
// A growing sequence writes its new tokens into the blocks it owns (possibly
// freshly allocated ones) and nothing already stored moves ("Ultimate Guide
// to PagedAttention", newline: KV cache and dynamic growth).  Token t goes to
// slot s = slot_mapping[t]: block s >> log2(bs), offset s & (bs - 1); K is a
// token-major row of the (block, kv-head) slab, V a column of its 16-token
// dimension-major sub-slab.  The copy is of raw bits.  One wavefront per (token, kv-head).  Also the
// whole-block copy that copy-on-write needs.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

template <typename W>  // W: uint16_t (bf16) or uint32_t (fp32) -- a raw element
__global__ __launch_bounds__(64) void kv_append_kernel(const AppendArgs a) {
  const int t = blockIdx.x / a.Hkv;
  const int h = blockIdx.x - t * a.Hkv;
  const int slot = a.slots[t];
  if (slot < 0) return;
  PA_DEVICE_CHECK((slot >> a.bs_log2) < a.num_blocks);
  const int bs = 1 << a.bs_log2;
  const int blk = slot >> a.bs_log2;
  const int off = slot & (bs - 1);
  const int D = a.D;
  const size_t slab = ((size_t)blk * a.Hkv + h) * (size_t)bs * D;  // elements
  const size_t src = ((size_t)t * a.Hkv + h) * D;
  const W* kn = static_cast<const W*>(a.k_new) + src;
  const W* vn = static_cast<const W*>(a.v_new) + src;
  W* kc = static_cast<W*>(a.k_cache) + slab + (size_t)off * D;  // row of the bs x D slab
  // column off % 16 of the D x 16 sub-slab off / 16
  W* vc = static_cast<W*>(a.v_cache) + slab + (size_t)(off >> 4) * D * 16 + (off & 15);
  for (int d = threadIdx.x; d < D; d += 64) {
    kc[d] = kn[d];
    vc[(size_t)d * 16] = vn[d];
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
  const long long blocks = (long long)a.T * a.Hkv;
  if (blocks <= 0) return hipSuccess;
  if (dtype == 1) {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3((unsigned)blocks), dim3(64), 0, s, a);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, dim3((unsigned)blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
