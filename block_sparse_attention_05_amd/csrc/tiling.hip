// Head-aware 3-D tiling for gfx950 (Veda page, section 2.2: each head tiles the token grid
// with its own factorisation (p_t, p_h, p_w) of the hardware tile, so that a block of
// consecutive tokens is a compact spatio-temporal cube).
//
// On a (T, Hg, W) grid with raster index n = (t*Hg + y)*W + x, the cube order of a head
// with cube (ct, ch, cw) sorts the tokens by (t/ct, y/ch, x/cw, t%ct, y%ch, x%cw). The
// position of token (t, y, x) in that order has a closed form: every cube before it in
// the cube grid is full along the axes where it precedes, so
//   pos = bt*ct*Hg*W + st*(by*ch*W + sy*bx*cw) + (it*sy + iy)*sx + ix
// with b* = cube coordinates, i* = offsets inside the cube and s* = this cube's extent
// along each axis (smaller on the far borders). The kernel walks tokens in raster order,
// so the raster side of the copy is coalesced; each thread moves one 16-byte granule.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

__device__ __forceinline__ int cube_pos(int n, int T, int Hg, int W, int ct, int ch, int cw) {
  const int x = n % W;
  const int ty = n / W;
  const int y = ty % Hg;
  const int t = ty / Hg;
  const int bt = t / ct, it = t - bt * ct, st = min(ct, T - bt * ct);
  const int by = y / ch, iy = y - by * ch, sy = min(ch, Hg - by * ch);
  const int bx = x / cw, ix = x - bx * cw, sx = min(cw, W - bx * cw);
  return bt * ct * Hg * W + st * (by * ch * W + sy * bx * cw) + (it * sy + iy) * sx + ix;
}

// grid (ceil(N * G / 256), B*H); G = 16-byte granules per row
__global__ __launch_bounds__(256) void cube_permute_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                           int H, int N, int G, int T, int Hg, int W,
                                                           CubeTable cubes, int inverse) {
  const int bh = blockIdx.y;
  const int h = bh % H;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)N * G) return;
  const int n = (int)(e / G);
  const int g = (int)(e - (long)n * G);
  const int p = cube_pos(n, T, Hg, W, cubes.c[h][0], cubes.c[h][1], cubes.c[h][2]);
  const size_t head = (size_t)bh * N * G;
  if (inverse)
    dst[head + (size_t)n * G + g] = src[head + (size_t)p * G + g];
  else
    dst[head + (size_t)p * G + g] = src[head + (size_t)n * G + g];
}

// order[h*N + pos_h(n)] = n, grid (ceil(N / 256), H)
__global__ __launch_bounds__(256) void cube_order_kernel(int N, int T, int Hg, int W, CubeTable cubes,
                                                         int32_t *__restrict__ order) {
  const int h = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int p = cube_pos(n, T, Hg, W, cubes.c[h][0], cubes.c[h][1], cubes.c[h][2]);
  order[(size_t)h * N + p] = n;
}

}  // namespace

hipError_t launch_cube_order(int H, int T, int Hg, int W, const CubeTable &cubes, int32_t *order,
                             hipStream_t s) {
  const int N = T * Hg * W;
  dim3 grid((unsigned)ceil_div(N, 256), H);
  cube_order_kernel<<<grid, 256, 0, s>>>(N, T, Hg, W, cubes, order);
  return hipGetLastError();
}

hipError_t launch_cube_permute(const void *src, void *dst, int BH, int H, int N, int row_bytes, int T,
                               int Hg, int W, const CubeTable &cubes, int inverse, hipStream_t s) {
  const int G = row_bytes / 16;
  const long total = (long)N * G;
  dim3 grid((unsigned)((total + 255) / 256), BH);
  cube_permute_kernel<<<grid, 256, 0, s>>>((const uint4 *)src, (uint4 *)dst, H, N, G, T, Hg, W, cubes, inverse);
  return hipGetLastError();
}

}  // namespace sa
