// kvq_append.hip — quantize new tokens' K/V rows and write them into their cache slots: one
// 64-lane wave per (token, KV head), the row quantizer of kvq_quant.h.  Every byte written
// belongs to its token alone, so concurrent tokens never touch the same byte.
#include "kvq_quant.h"

namespace kvq {
namespace {

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long long)a.n_tok * a.num_kv_heads) return;
  const int n = (int)(item / a.num_kv_heads);
  const int h = (int)(item % a.num_kv_heads);
  const long long slot = a.slots[n];
  const int P = a.page_size;
  if (slot < 0 || slot >= (long long)a.num_pages * P) return;  // padding / out of pool: skip
  const int page = (int)(slot / P), s = (int)(slot % P);
  uint8_t* blk = a.pool + ((size_t)page * a.num_kv_heads + h) * block_bytes(P, D);
  const size_t row = ((size_t)n * a.num_kv_heads + h) * D;
  append_row<D>(blk, P, s, a.k + row, a.v + row, lane);
}

}  // namespace

hipError_t launch_append(int head_dim, const AppendArgs& a, hipStream_t stream) {
  const long long items = (long long)a.n_tok * a.num_kv_heads;
  const unsigned grid = (unsigned)((items + 3) / 4);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(append_kernel<64>, dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(append_kernel<128>, dim3(grid), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(append_kernel<256>, dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
