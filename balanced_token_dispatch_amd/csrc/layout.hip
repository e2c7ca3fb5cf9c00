// moe_dispatch_layout: plan -> cu_seqlens of one rank, the destination row of
// every token copy, and that rank's receive map.
//
// Pages: ainovat.com "Moonshot AI Open-Sources MoonEP", contract paragraph
// (dispatch returns a cu_seqlens over the E+B weight rows that selects the
// active rows) and contiguity paragraph (experts addressed by row index);
// moses-y.github.io "MoonEP", "What This Does" (tokens written straight to
// their final expert-grouped position).
//
// The destination of copy c with expert e is fixed by g = its position among
// e's copies in copy-id order (a stable counting sort key).  Three launches:
//   k_lay_hist     grid (chunks, R): per-chunk expert histogram, stored
//                  expert-major so the next pass scans one contiguous row
//   k_lay_scan     grid E+1: block e < E scans its row over all (rank, chunk)
//                  -> first g of expert e in every chunk; block E builds the
//                  per-expert home offsets, every replica's destination base,
//                  this rank's cu_seqlens, and clears the unused src_flat tail
//   k_lay_scatter  grid (chunks, R): stable in-chunk rank of every copy from
//                  wave ballots (64-lane peer masks built bit by bit over the
//                  expert id) and per-wave LDS counters, then dest_pos and,
//                  for copies landing on this rank, src_flat
#include "common.hpp"

namespace moe {

// Chunk of one rank's copies per block, and block size.  In k_lay_scatter each wave walks
// kLayChunk / kLayWaves copies one wavefront at a time (a dependent chain of ballots and LDS
// counter updates), so that length sets its latency: 2048 copies on 8 waves (256 per wave)
// measured 28 us for the whole layout at R32 S4096 K8, against 52 us for 4096 on 4 waves.
constexpr int kLayChunk = 2048;
constexpr int kLayThreads = 512;
constexpr int kLayWaves = kLayThreads / kWave;
constexpr int kLayMaxE = 1024;
constexpr int kLayMaxL = 1024 + 512;

__global__ __launch_bounds__(kLayThreads) void k_lay_hist(const int32_t *__restrict__ topk,
                                                          int32_t *__restrict__ part, int SK,
                                                          int E, int nchunk, int npc) {
  __shared__ int hist[kLayMaxE];
  const int c = blockIdx.x, p = blockIdx.y;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int lo = c * kLayChunk, hi = min(SK, lo + kLayChunk);
  const int32_t *ids = topk + (size_t)p * SK;
  // all of a thread's ids are loaded before the first is counted, so the loads overlap
  constexpr int kPer = kLayChunk / kLayThreads;
  int ev[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = lo + u * kLayThreads + threadIdx.x;
    ev[u] = i < hi ? ids[i] : -1;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (ev[u] >= 0 && ev[u] < E) atomicAdd(&hist[ev[u]], 1);
  __syncthreads();
  const int col = p * nchunk + c;
  for (int e = threadIdx.x; e < E; e += blockDim.x) part[(size_t)e * npc + col] = hist[e];
}

// Exclusive scan of one int per thread over a kLayThreads-thread block (kLayWaves waves).
__device__ int lay_block_scan_excl(int v, int *tmp /* >= kLayWaves */, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kLayWaves; ++w) {
    const int t = tmp[w];
    base += (w < wid) ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return base + x - v;
}

__global__ __launch_bounds__(kLayThreads) void k_lay_scan(
    int32_t *__restrict__ part, const int32_t *__restrict__ plan, int32_t *__restrict__ hs,
    int32_t *__restrict__ rdst, int32_t *__restrict__ cu_out, int32_t *__restrict__ src_flat,
    int npc, int R, int S, int K, int E, int B, int rank) {
  __shared__ int tmp[kLayWaves];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  const int SK = S * K;
  const int E_loc = E / R;
  const PlanLayout L(E, R, B);
  if ((int)blockIdx.x < E) {
    // exclusive scan of expert e's chunk counts over (rank, chunk) in order
    int32_t *row = part + (size_t)blockIdx.x * npc;
    int carry = 0;
    for (int base = 0; base < npc; base += kLayThreads) {
      const int i = base + tid;
      const int v = i < npc ? row[i] : 0;
      int total;
      const int ex = lay_block_scan_excl(v, tmp, &total);
      if (i < npc) row[i] = carry + ex;
      carry += total;
    }
    return;
  }
  // block E: tables that depend on the plan only
  const int nRep = plan[1];
  for (int e = tid; e < E; e += kLayThreads) {
    const int r0 = (e / E_loc) * E_loc;
    int s = 0;
#pragma unroll 8
    for (int f = r0; f < e; ++f) s += plan[L.off_keep + f];
    hs[e] = s;
  }
  for (int m = tid; m < nRep && m < E + R; m += kLayThreads) {
    const int slot = plan[L.off_rslot + m];
    int d = -1;
    if (slot >= 0) {
      const int q = plan[L.off_rrank + m];
      int pos = 0;
      for (int f = q * E_loc; f < (q + 1) * E_loc; ++f) pos += plan[L.off_keep + f];
      for (int j = 0; j < slot; ++j) pos += plan[L.off_scount + q * B + j];
      d = q * SK + pos;
    }
    rdst[m] = d;
  }
  // cu_seqlens of `rank`: rows of its home experts, then its slots
  const int G = E + B;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < G; base += kLayThreads) {
    const int rho = base + tid;
    int n = 0;
    if (rho < E)
      n = (rho / E_loc == rank) ? plan[L.off_keep + rho] : 0;
    else if (rho < G)
      n = plan[L.off_scount + rank * B + (rho - E)];
    int total;
    const int ex = lay_block_scan_excl(n, tmp, &total);
    const int carry = carry_s;
    if (rho < G) cu_out[rho] = carry + ex;
    __syncthreads();
    if (tid == 0) carry_s = carry + total;
    __syncthreads();
  }
  const int filled = carry_s;
  if (tid == 0) cu_out[G] = filled;
  for (int i = filled + tid; i < SK; i += kLayThreads) src_flat[i] = -1;
}

__global__ __launch_bounds__(kLayThreads) void k_lay_scatter(
    const int32_t *__restrict__ topk, const int32_t *__restrict__ part,
    const int32_t *__restrict__ plan, const int32_t *__restrict__ hs,
    const int32_t *__restrict__ rdst, int32_t *__restrict__ dest_pos,
    int32_t *__restrict__ src_flat, int nchunk, int npc, int R, int S, int K, int E, int B,
    int rank, int nbits) {
  __shared__ int sIds[kLayChunk];
  __shared__ int sBase[kLayWaves][kLayMaxE];
  __shared__ int sKeep[kLayMaxE], sHs[kLayMaxE], sRepFirst[kLayMaxE], sRepN[kLayMaxE];
  __shared__ int sRstart[kLayMaxL], sRcount[kLayMaxL], sRdst[kLayMaxL];

  const int c = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int SK = S * K;
  const int E_loc = E / R;
  const PlanLayout L(E, R, B);
  const int lo = c * kLayChunk;
  const int len = min(SK - lo, kLayChunk);
  const int32_t *ids = topk + (size_t)p * SK + lo;

  for (int i = tid; i < len; i += kLayThreads) {
    const int e = ids[i];
    sIds[i] = (e >= 0 && e < E) ? e : E;
  }
  for (int e = tid; e < E; e += kLayThreads) {
    sKeep[e] = plan[L.off_keep + e];
    sHs[e] = hs[e];
    sRepFirst[e] = plan[L.off_rep_first + e];
    sRepN[e] = plan[L.off_rep_n + e];
#pragma unroll
    for (int w = 0; w < kLayWaves; ++w) sBase[w][e] = 0;
  }
  const int nRep = min(plan[1], E + R);
  for (int m = tid; m < nRep; m += kLayThreads) {
    sRstart[m] = plan[L.off_rstart + m];
    sRcount[m] = plan[L.off_rcount + m];
    sRdst[m] = rdst[m];
  }
  __syncthreads();

  // each of the kLayWaves waves owns a contiguous 1/kLayWaves of the chunk
  const int per_wave = kLayChunk / kLayWaves;
  const int w0 = wid * per_wave;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  auto peers_of = [&](int key, bool valid) -> uint64_t {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bm = __ballot(bit);
      m &= bit ? bm : ~bm;
    }
    return valid ? m : 0ull;
  };

  // pass 1: per-wave expert counts
  for (int it = 0; it < per_wave; it += kWave) {
    const int i = w0 + it + lane;
    const bool valid = i < len;
    const int key = valid ? sIds[i] : E;
    const uint64_t peers = peers_of(key, valid);
    const bool leader = valid && key < E && (peers & lt_mask) == 0;
    if (leader) sBase[wid][key] += __popcll(peers);
  }
  __syncthreads();
  // per-wave starting g: chunk offset from the scan plus earlier waves' counts
  const int col = p * nchunk + c;
  for (int e = tid; e < E; e += kLayThreads) {
    int run = part[(size_t)e * npc + col];
#pragma unroll
    for (int w = 0; w < kLayWaves; ++w) {
      const int t = sBase[w][e];
      sBase[w][e] = run;
      run += t;
    }
  }
  __syncthreads();
  // pass 2: g of every copy, then its destination
  for (int it = 0; it < per_wave; it += kWave) {
    const int i = w0 + it + lane;
    const bool valid = i < len;
    const int key = valid ? sIds[i] : E;
    const uint64_t peers = peers_of(key, valid);
    int g = 0;
    if (valid && key < E) {
      g = sBase[wid][key] + __popcll(peers & lt_mask);
    }
    const bool leader = valid && key < E && (peers & lt_mask) == 0;
    if (leader) sBase[wid][key] += __popcll(peers);
    if (!valid) continue;
    int dest = -1;
    if (key < E) {
      if (g < sKeep[key]) {
        dest = (key / E_loc) * SK + sHs[key] + g;
      } else {
        const int f = sRepFirst[key], n = sRepN[key];
        for (int m = f; m < f + n; ++m) {
          const int st = sRstart[m];
          if (g >= st && g < st + sRcount[m]) {
            if (sRdst[m] >= 0) dest = sRdst[m] + (g - st);
            break;
          }
        }
      }
    }
    const int copy = p * SK + lo + i;
    dest_pos[copy] = dest;
    if (dest >= rank * SK && dest < (rank + 1) * SK) src_flat[dest - rank * SK] = copy;
  }
}

}  // namespace moe

using namespace moe;

static int lay_nchunk(const moe_dims *d) { return ceil_div((long long)d->S * d->K, kLayChunk); }

extern "C" size_t moe_dispatch_layout_workspace_bytes(const moe_dims *d) {
  if (!dims_ok(d)) return 0;
  const size_t npc = (size_t)d->R * lay_nchunk(d);
  return (npc * d->E + d->E + (d->E + d->R)) * sizeof(int32_t);
}

extern "C" moe_status_t moe_dispatch_layout(const moe_dims *d, int32_t rank,
                                            const int32_t *topk_idx, const int32_t *plan,
                                            int32_t *cu_seqlens, int32_t *dest_pos,
                                            int32_t *src_flat, void *ws, size_t ws_bytes,
                                            hipStream_t stream) {
  if (!dims_ok(d) || !topk_idx || !plan || !cu_seqlens || !dest_pos || !src_flat || !ws)
    return MOE_EINVAL;
  if (rank < 0 || rank >= d->R) return MOE_EINVAL;
  if (ws_bytes < moe_dispatch_layout_workspace_bytes(d)) return MOE_ENOSPACE;
  const int SK = d->S * d->K;
  const int nchunk = lay_nchunk(d);
  const int npc = d->R * nchunk;
  int32_t *part = (int32_t *)ws;
  int32_t *hs = part + (size_t)npc * d->E;
  int32_t *rdst = hs + d->E;
  int nbits = 1;
  while ((1 << nbits) <= d->E) ++nbits;  // keys 0..E (E = no destination) fit in nbits
  hipLaunchKernelGGL(k_lay_hist, dim3(nchunk, d->R), dim3(kLayThreads), 0, stream, topk_idx,
                     part, SK, d->E, nchunk, npc);
  hipLaunchKernelGGL(k_lay_scan, dim3(d->E + 1), dim3(kLayThreads), 0, stream, part, plan, hs,
                     rdst, cu_seqlens, src_flat, npc, d->R, d->S, d->K, d->E, d->B, rank);
  hipLaunchKernelGGL(k_lay_scatter, dim3(nchunk, d->R), dim3(kLayThreads), 0, stream, topk_idx,
                     part, plan, hs, rdst, dest_pos, src_flat, nchunk, npc, d->R, d->S, d->K,
                     d->E, d->B, rank, nbits);
  return launch_status();
}
