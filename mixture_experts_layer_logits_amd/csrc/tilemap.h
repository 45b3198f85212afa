// Device-side tile map shared by the grouped GEMM kernels.  Group boundaries (the expert
// offsets) live only on the device; every workgroup rebuilds the map in LDS from them
// and walks a persistent, XCD-aware schedule over it.
//
//   Group::M  rows grouped by expert: the M-tiles of expert e are numbered from
//             s_map[e] = sum_{e' < e} ceil(rows_e' / BM); its tiles are numbered N-tile
//             major (consecutive tiles read the same weight block) or, for problems that
//             set N_MAJOR = false, M-tile major (consecutive tiles read the same rows).
//   Group::K  reduction grouped by expert: one output tile set per expert, experts
//             ordered by descending row count (ties: lower id) so the longest reductions
//             start first.
#pragma once
#include "common.h"
#include "gemm.h"

namespace moe {

struct TileRange {
  int e, m0, m_end, n0, k_beg, k_end;
};

// seg(e): start row of group e (e in [0, E]).  Returns the number of tiles.
template <Group GROUP, int BM, int BN, int NT, class Seg>
__device__ __forceinline__ int build_tile_map(int* s_map, Seg seg, int E, int M, int N, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int ntn = (N + BN - 1) / BN;
  if constexpr (GROUP == Group::M) {
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < E; base += kWave) {
        const int e = base + lane;
        const int x = e < E ? (seg(e + 1) - seg(e) + BM - 1) / BM : 0;
        int incl = x;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += y;
        }
        if (e < E) s_map[e] = carry + incl - x;
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) s_map[E] = carry;
    }
    __syncthreads();
    return s_map[E] * ntn;
  } else {
    for (int e = tid; e < E; e += NT) {
      const int ce = seg(e + 1) - seg(e);
      int rank = 0;
      for (int o = 0; o < E; o++) {
        const int co = seg(o + 1) - seg(o);
        rank += (co > ce) || (co == ce && o < e);
      }
      s_map[rank] = e;
    }
    __syncthreads();
    return E * ((M + BM - 1) / BM) * ntn;
  }
}

// Tile t of the map.  Group::M: K range [0, K); Group::K: K range = the expert's rows.
// NMAJOR (Group::M): an expert's tiles are numbered N-tile major, else M-tile major.
template <Group GROUP, int BM, int BN, bool NMAJOR, class Seg>
__device__ __forceinline__ TileRange tile_at(int t, const int* s_map, Seg seg, int E, int M, int N, int K) {
  const int ntn = (N + BN - 1) / BN;
  TileRange r;
  if constexpr (GROUP == Group::M) {
    // expert e owns tiles [s_map[e] * ntn, s_map[e + 1] * ntn).  N-tile major: the M-tiles
    // that read the same weight block are consecutive, so a run of tiles that ends inside
    // an expert splits it between N-tiles (each weight block still read by one run) rather
    // than between M-tiles (every weight block read by both runs).
    const int mt = t / ntn;
    int lo = 0, hi = E;  // largest e with s_map[e] <= mt
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_map[mid] <= mt) lo = mid; else hi = mid;
    }
    r.e = lo;
    if constexpr (NMAJOR) {
      const int me = s_map[lo + 1] - s_map[lo];  // M-tiles of expert lo (>= 1 here)
      const int local = t - s_map[lo] * ntn;
      const int nt = local / me;
      r.n0 = nt * BN;
      r.m0 = seg(lo) + (local - nt * me) * BM;
    } else {
      r.n0 = (t % ntn) * BN;
      r.m0 = seg(lo) + (mt - s_map[lo]) * BM;
    }
    r.m_end = seg(lo + 1);
    r.k_beg = 0;
    r.k_end = K;
  } else {
    const int mtn = (M + BM - 1) / BM;
    const int per_e = mtn * ntn;
    r.e = s_map[t / per_e];
    const int rem = t % per_e;
    r.m0 = (rem / ntn) * BM;
    r.n0 = (rem % ntn) * BN;
    r.m_end = M;
    r.k_beg = seg(r.e);
    r.k_end = seg(r.e + 1);
  }
  return r;
}

// Logical workgroup id: hardware places workgroup b on XCD b % 8; this numbering gives
// each XCD a contiguous run of logical ids, so tiles that share operands share an L2.
__device__ __forceinline__ int xcd_logical_wg() {
  const int G = gridDim.x;
  return (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
}

}  // namespace moe
