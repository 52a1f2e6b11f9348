// Geometry lookup tables for the gather paths of the backward kernels.
//
// The tiling (block-row-major [block_t, block_h, block_w] blocks with smaller
// edge blocks) needs integer divisions by runtime sizes to map (block, row)
// to a token.  The matrix-core kernels gather 16-byte chunks of many rows per
// step, so they read these precomputed tables instead: one small launch per
// call fills them in the caller's workspace.  (The forward places its rows
// by arithmetic once per workgroup and launches no table kernel.)
#include "common.h"

namespace pbsa {
namespace {

__global__ __launch_bounds__(256) void geo_table_kernel(Geo g, int32_t* btok, int32_t* blen, int32_t* pbase,
                                                        int32_t* pblk) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx < g.nq * g.C) {
    const int j = idx / g.C, r = idx - j * g.C;
    const BlockExt e = block_ext(g, j);
    btok[idx] = r < e.len ? block_token(g, e, r) : -1;
    if (r == 0) blen[j] = e.len;
  }
  if (idx < g.nl) {
    pbase[idx] = (idx / g.nq) * g.ct;
    pblk[idx] = idx % g.nq;
  }
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t geo_table_bytes(const Geo& g) {
  return a256((size_t)g.nq * g.C * 4) + a256((size_t)g.nq * 4) + 2 * a256((size_t)g.nl * 4);
}

hipError_t launch_geo_table(const Geo& g, void* ws, GeoTab* tab, hipStream_t s) {
  char* p = (char*)ws;
  int32_t* btok = (int32_t*)p;
  p += a256((size_t)g.nq * g.C * 4);
  int32_t* blen = (int32_t*)p;
  p += a256((size_t)g.nq * 4);
  int32_t* pbase = (int32_t*)p;
  p += a256((size_t)g.nl * 4);
  int32_t* pblk = (int32_t*)p;
  tab->btok = btok;
  tab->blen = blen;
  tab->pbase = pbase;
  tab->pblk = pblk;
  const int n = g.nq * g.C > g.nl ? g.nq * g.C : g.nl;
  geo_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(g, btok, blen, pbase, pblk);
  return hipGetLastError();
}

}  // namespace pbsa
