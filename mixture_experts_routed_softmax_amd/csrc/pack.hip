// Packing of expert weights into the tile-contiguous layout the packed grouped
// GEMMs stream (a one-time transform at model load, not part of a forward).
//
// The weights arrive as nn.Linear matrices [E, N, K] (K contiguous).  A GEMM
// tile covers 256 weight rows and advances through K in steps of 64 bytes
// (32 bf16 or 64 fp8 codes).  Row-major storage makes every step read 64
// bytes from each of 256 rows that are K*elt bytes apart, which HBM serves
// far below its peak.  The packed layout stores, for every expert e, row tile
// nt and K step kt, one contiguous 16 KB chunk
//     chunk(e, nt, kt) at byte ((e * NT + nt) * KT + kt) * 16384
// whose byte row*64 + p*16 holds the 16 bytes of tile row `row` at K bytes
// kt*64 + c*16 with c = p ^ ((row >> 2) & 3): exactly the LDS image of one
// pipeline stage, so a stage is one contiguous 1 KB-per-wave DMA.
//   gate/up: tile nt rows 0..127 = w_gate channels nt*128 .., rows 128..255 =
//            the same channels of w_up (NT = ceil(I / 128))
//   down:    tile nt rows = w_down output channels nt*256 .. (NT = ceil(H / 256))
// Rows past N are zero.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ w0,
                                                   const uint8_t* __restrict__ w1, int gate_up,
                                                   int N, int64_t row_bytes, int NT, int KT,
                                                   int64_t total_chunks16, uint8_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-byte unit of the output
  if (i >= total_chunks16) return;
  const int64_t chunk = i >> 10;        // 1024 units of 16 B per 16 KB chunk
  const int unit = (int)(i & 1023);
  const int row = unit >> 2;
  const int p = unit & 3;
  const int c = p ^ ((row >> 2) & 3);
  const int kt = (int)(chunk % KT);
  const int64_t et = chunk / KT;
  const int nt = (int)(et % NT);
  const int64_t e = et / NT;
  int n;
  const uint8_t* src;
  if (gate_up) {
    n = nt * 128 + (row & 127);
    src = row < 128 ? w0 : w1;
  } else {
    n = nt * 256 + row;
    src = w0;
  }
  i32x4 v = {0, 0, 0, 0};
  if (n < N) v = *(const i32x4*)(src + (e * N + n) * row_bytes + (int64_t)kt * 64 + c * 16);
  *(i32x4*)(dst + i * 16) = v;
}

}  // namespace

int64_t packed_tiles(int which_gate_up, int N) {
  return which_gate_up ? (N + 127) / 128 : (N + 255) / 256;
}

hipError_t launch_pack(const void* w0, const void* w1, int gate_up, int E, int N, int64_t row_bytes,
                       void* dst, hipStream_t stream) {
  const int NT = (int)packed_tiles(gate_up, N);
  const int KT = (int)(row_bytes / 64);
  const int64_t units = (int64_t)E * NT * KT * 1024;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                     (const uint8_t*)w0, (const uint8_t*)w1, gate_up, N, row_bytes, NT, KT, units,
                     (uint8_t*)dst);
  return hipGetLastError();
}

}  // namespace moe
