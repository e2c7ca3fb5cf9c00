// moe_plan: per-expert histogram of all ranks' router outputs and the
// greedy redundant-expert placement that gives every rank exactly S*K copies.
//
// Pages: ainovat.com "Moonshot AI Open-Sources MoonEP", paragraphs on the
// skew metric (per-expert token counts), the exact S*K-per-rank invariant and
// the mechanism (a few redundant experts planned online from the current
// router outputs); findrepo.work "MoonEP" card, "Strengths" (near-optimal
// choice, negligible planning cost).  The placement rule itself is this
// library's reading; it is spelled out at moe_plan in moe.h.
//
// Three launches, no atomics on global memory, so the result is
// deterministic:
//   k_plan_hist    grid (chunks, R): LDS histogram of 4096 ids -> partials
//   k_plan_reduce  grid R: sum the partials of one rank -> counts[p][*]
//   k_plan_solve   one 1024-thread workgroup: loads, donor/receiver order,
//                  pieces, the piece/receiver walk and slots, all as
//                  counting ranks and block scans in LDS (no serial loop
//                  over ranks or experts).  Only when some receiver would
//                  need more than B slots, one thread then re-places the
//                  walk's replicas with the relay fallback (relay_pass) and
//                  the block regroups the list by expert.
#include <climits>
#include <mutex>

#include "common.hpp"

namespace moe {

constexpr int kPlanChunk = 4096;
constexpr int kHistThreads = 1024;  // 4 ids per thread: 35 -> 30 us per plan against 256 threads
constexpr int kSolveThreads = 1024;
constexpr int kMaxE = 1024;
constexpr int kMaxR = 512;
constexpr int kMaxL = kMaxE + kMaxR;

// ids of rank p, chunk c -> partial[(p*nchunk + c)*(E+1) + e]; bin E counts bad ids.
__global__ __launch_bounds__(kHistThreads) void k_plan_hist(const int32_t *__restrict__ topk,
                                                            int32_t *__restrict__ partial, int SK,
                                                            int E, int nchunk) {
  __shared__ int hist[kMaxE + 1];
  const int c = blockIdx.x, p = blockIdx.y;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int lo = c * kPlanChunk;
  const int hi = min(SK, lo + kPlanChunk);
  const int32_t *ids = topk + (size_t)p * SK;
  // all of a thread's ids are loaded before the first is counted (kPlanChunk / kHistThreads
  // per thread), so the loads overlap instead of each waiting for the one before
  constexpr int kPer = kPlanChunk / kHistThreads;
  int ev[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = lo + u * blockDim.x + threadIdx.x;
    ev[u] = i < hi ? ids[i] : 0;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (lo + u * (int)blockDim.x + (int)threadIdx.x >= hi) continue;
    const int e = ev[u];
    const int key = (e >= 0 && e < E) ? e : E;
    atomicAdd(&hist[key], 1);
  }
  __syncthreads();
  int32_t *dst = partial + (size_t)(p * nchunk + c) * (E + 1);
  for (int e = threadIdx.x; e <= E; e += blockDim.x) dst[e] = hist[e];
}

// counts[p][e] = sum over chunks; bad[p] = number of bad ids of rank p.
__global__ __launch_bounds__(kHistThreads) void k_plan_reduce(const int32_t *__restrict__ partial,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ bad, int E,
                                                              int nchunk) {
  const int p = blockIdx.x;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    int s = 0;
#pragma unroll 8
    for (int c = 0; c < nchunk; ++c) s += partial[(size_t)(p * nchunk + c) * (E + 1) + e];
    if (e < E)
      counts[(size_t)p * E + e] = s;
    else
      bad[p] = s;
  }
}

// Exclusive scan of one int per thread across a 1024-thread workgroup.
__device__ int block_scan_excl(int v, int *tmp /* >= 17 ints */, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const int nw = blockDim.x >> 6;
    int w = lane < nw ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < nw) tmp[lane] = w;  // inclusive per-wave totals
  }
  __syncthreads();
  const int base = wid ? tmp[wid - 1] : 0;
  *total = tmp[(blockDim.x >> 6) - 1];
  __syncthreads();
  return base + x - v;
}

// Relay fallback state, all in LDS: the replica list (edited in place: the
// pass writes entry w while reading walk entry m >= w, each walk entry giving
// at most one new entry), copies kept home, and per rank its slot count and
// its replicas as a chain in slot order.
struct RelayState {
  int *rexp, *rrank, *rcount, *rslot;
  int *keep, *hosted, *chain_first, *chain_last, *chain_next;
  int E_loc, B;
  int w;

  __device__ int entry_of(int a, int e) const {
    for (int i = chain_first[a]; i >= 0; i = chain_next[i])
      if (rexp[i] == e) return i;
    return -1;
  }
  __device__ bool can_place(int e, int a) const {
    return a == e / E_loc || entry_of(a, e) >= 0 || hosted[a] < B;
  }
  __device__ void append(int e, int a, int n, int slot) {
    rexp[w] = e;
    rrank[w] = a;
    rcount[w] = n;
    rslot[w] = slot;
    if (slot >= 0) {
      chain_next[w] = -1;
      if (chain_last[a] >= 0) chain_next[chain_last[a]] = w; else chain_first[a] = w;
      chain_last[a] = w;
      ++hosted[a];
    }
    ++w;
  }
  // n copies of e onto rank a: home, an existing replica, or a new slot
  __device__ void place(int e, int a, int n) {
    if (a == e / E_loc) {
      keep[e] += n;
      return;
    }
    const int i = entry_of(a, e);
    if (i >= 0) rcount[i] += n; else append(e, a, n, hosted[a]);
  }
};

// One thread.  For each walk replica (f, q, x) in emission order: place it on
// q; else relay through one of q's replicas (e, c) in slot order (q takes x
// more copies of e from keep_e, e's home takes the x copies of f); else
// switch one of them (it becomes f with c + x copies, c taken from keep_f,
// and f's home takes the c copies of e); else drop it.  Returns the number
// of relayed or switched replicas; *dropped counts the dropped ones.
__device__ int relay_pass(RelayState &st, int nWalk, int *dropped) {
  int relayed = 0, nd = 0;
  st.w = 0;
  for (int m = 0; m < nWalk; ++m) {
    const int f = st.rexp[m], q = st.rrank[m], x = st.rcount[m];
    if (st.can_place(f, q)) {
      st.place(f, q, x);
      continue;
    }
    bool done = false;
    for (int i = st.chain_first[q]; i >= 0 && !done; i = st.chain_next[i]) {
      const int e = st.rexp[i], A = e / st.E_loc;
      if (st.keep[e] >= x && st.can_place(f, A)) {
        st.rcount[i] += x;
        st.keep[e] -= x;
        st.place(f, A, x);
        done = true;
      }
    }
    for (int i = st.chain_first[q]; i >= 0 && !done; i = st.chain_next[i]) {
      const int e = st.rexp[i], c = st.rcount[i], F = f / st.E_loc;
      if (st.keep[f] >= c && st.can_place(e, F)) {
        st.rexp[i] = f;
        st.rcount[i] = c + x;
        st.keep[f] -= c;
        st.place(e, F, c);
        done = true;
      }
    }
    if (done) {
      ++relayed;
    } else {
      st.append(f, q, x, -1);
      ++nd;
    }
  }
  *dropped = nd;
  return relayed;
}

// Second fallback, run only when relay_pass drops a replica and B >= 1: a bounded depth-first
// search for a plan with at most one replica per rank, in generations.  Generation 0 is the
// receivers, each needing -d_r copies; each rank of a generation, by (need desc, r asc), takes
// its whole need from one expert f whose home g has taken no copies and is not in the
// generation, with cap_f >= need (cap starts at T); experts are tried in a fixed order (homes
// by (d desc, r asc), a home's experts by (T desc, e asc)), first those whose home has that
// much excess left (d_g - out_g >= need), then the others.  When a generation is placed, the
// ranks that took no copies and sent out more than their excess form the next one, each
// needing out_r - d_r; with none left the plan is complete if every such rank sent out exactly
// its excess.  A failed continuation undoes the last choice and tries the next candidate; at
// most kSearchBudget placements are tried.  One wavefront runs it: its 64 lanes test 64
// candidates at a time and the first that fits is taken, so the order is the serial one.
// The state is in LDS, each word written by one lane and read by any lane of the same
// wavefront, whose LDS accesses take effect in program order; the pointers to what changes
// are volatile so that every access is made where the code makes it.
constexpr int kSearchBudget = 512;
constexpr int kTaken = INT_MIN;  // avail[] of a rank that takes copies

struct SearchState {
  const int *cand;      // [E] experts in trial order
  const int *cand_g;    // [E] their homes
  volatile int *cap;    // [E] copies of e not yet placed elsewhere
  volatile int *out;    // [R] copies rank r has sent out
  volatile int *avail;  // [R] d_r - out_r, or kTaken if r takes copies
  volatile int *pn;     // [R] ranks of the generations, in order
  volatile int *pneed;  // [R] their needs
  volatile int *gs;     // [R+1] first position of each generation, and the end
  volatile int *ci;     // [R] candidate taken at each position
  const int *D;         // excess per rank
  int E, R;
};

// First candidate position c >= c0 that a rank needing `need` copies can take: c < E is
// cand[c] with a home that has that much excess left, E <= c < 2E is cand[c - E] with a home
// that has not.  2E if none.  One sweep over the candidates answers both passes (each
// candidate is in exactly one of them), stopping at the first fitting candidate at or past c0.
// Wave-uniform.
__device__ int search_scan(const SearchState &s, int c0, int need, int lane) {
  const int k0 = c0 < s.E ? c0 : c0 - s.E;  // first candidate of the pass c0 is in
  int other = 2 * s.E;
  for (int base = 0; base < s.E; base += 64) {
    const int k = base + lane;
    bool fit = false, oth = false;
    if (k < s.E) {
      const int a = s.avail[s.cand_g[k]];
      if (a != kTaken && s.cap[s.cand[k]] >= need) {
        fit = a >= need && c0 < s.E && k >= k0;
        oth = a < need && (c0 < s.E || k >= k0);
      }
    }
    const unsigned long long mf = __ballot(fit);
    if (mf) return base + __ffsll((unsigned long long)mf) - 1;
    const unsigned long long mo = __ballot(oth);
    if (mo && other == 2 * s.E) other = s.E + base + __ffsll((unsigned long long)mo) - 1;
  }
  return other;
}

// One wavefront (all 64 lanes).  s.pn/pneed[0, n0) hold generation 0, marked taken in avail,
// and s.gs[0..1] = 0, n0.  Returns the number of placements of a complete plan (positions
// 0..n-1 of pn, pneed, ci), or -1; *steps = placements tried.
__device__ int relay_search(const SearchState &s, int n0, int lane, int *steps) {
  int i = 0, g = 0, gend = n0, c0 = 0;
  *steps = 0;
  for (;;) {
    bool back = false;
    if (i == gend) {
      // the next generation: ranks that take no copies and sent out more than their excess,
      // gathered in rank order, then put in (need desc, r asc) order
      int cnt = 0;
      bool balanced = true;
      for (int r0 = 0; r0 < s.R; r0 += 64) {
        const int r = r0 + lane;
        const int a = r < s.R ? s.avail[r] : kTaken;
        const bool over = a != kTaken && a < 0;
        const unsigned long long m = __ballot(over);
        if (over) {
          const int j = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                  (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          s.pn[gend + j] = r;
          s.pneed[gend + j] = -a;
        }
        cnt += __popcll(m);
        balanced = balanced && __ballot(a != kTaken && a != 0) == 0;
      }
      if (cnt == 0) {
        if (balanced) return gend;
        back = true;
      } else {
        // every entry's place among the cnt entries, all read before any is moved
        constexpr int kPer = kMaxR / 64;
        int rr[kPer], nn[kPer], pp[kPer];
#pragma unroll
        for (int b = 0; b < kPer; ++b) {
          const int t = lane + 64 * b;
          rr[b] = t < cnt ? s.pn[gend + t] : 0;
          nn[b] = t < cnt ? s.pneed[gend + t] : 0;
        }
#pragma unroll
        for (int b = 0; b < kPer; ++b) {
          int pos = 0;
          if (lane + 64 * b < cnt)
            for (int u = 0; u < cnt; ++u) {
              const int nu = s.pneed[gend + u], ru = s.pn[gend + u];
              pos += nu > nn[b] || (nu == nn[b] && ru < rr[b]);
            }
          pp[b] = pos;
        }
#pragma unroll
        for (int b = 0; b < kPer; ++b)
          if (lane + 64 * b < cnt) {
            s.pn[gend + pp[b]] = rr[b];
            s.pneed[gend + pp[b]] = nn[b];
            s.avail[rr[b]] = kTaken;
          }
        ++g;
        gend += cnt;
        if (lane == 0) s.gs[g + 1] = gend;
        c0 = 0;
        continue;
      }
    }
    if (!back) {
      const int need = s.pneed[i];
      const int c = search_scan(s, c0, need, lane);
      if (c < 2 * s.E) {
        if (*steps == kSearchBudget) return -1;
        ++*steps;
        const int k = c < s.E ? c : c - s.E;
        const int f = s.cand[k], h = s.cand_g[k];
        if (lane == 0) {
          s.cap[f] = s.cap[f] - need;
          s.out[h] = s.out[h] + need;
          s.avail[h] = s.D[h] - s.out[h];
          s.ci[i] = c;
        }
        ++i;
        c0 = 0;
        continue;
      }
    }
    // no (further) candidate here: undo the previous placement and try its next candidate,
    // first dropping the current generation if this is its first position
    if (g > 0 && i == s.gs[g]) {
      for (int p = s.gs[g] + lane; p < gend; p += 64) {
        const int r = s.pn[p];
        s.avail[r] = s.D[r] - s.out[r];
      }
      --g;
      gend = s.gs[g + 1];
    }
    if (i == 0) return -1;
    --i;
    const int c = s.ci[i], need = s.pneed[i];
    const int k = c < s.E ? c : c - s.E;
    const int f = s.cand[k], h = s.cand_g[k];
    if (lane == 0) {
      s.cap[f] = s.cap[f] + need;
      s.out[h] = s.out[h] - need;
      s.avail[h] = s.D[h] - s.out[h];
    }
    c0 = c + 1;
  }
}

__global__ __launch_bounds__(kSolveThreads) void k_plan_solve(const int32_t *__restrict__ counts,
                                                              const int32_t *__restrict__ bad,
                                                              int32_t *__restrict__ plan,
                                                              uint32_t *__restrict__ dev_status,
                                                              int R, int S, int K, int E, int B) {
  // per expert
  __shared__ int sT[kMaxE], sKeep[kMaxE], sSrank[kMaxE], sPre[kMaxE], sA[kMaxE];
  __shared__ int sRepFirst[kMaxE], sRepN[kMaxE];
  // per piece (indexed by global piece order, at most E pieces)
  __shared__ int sPieceE[kMaxE], sPieceP[kMaxE], sPieceJlo[kMaxE], sPieceCnt[kMaxE];
  // per rank
  __shared__ int sD[kMaxR], sDonorPos[kMaxR], sDonorAt[kMaxR], sRecvAt[kMaxR], sNP[kMaxR];
  __shared__ int sDonorBase[kMaxR], sPieceBase0[kMaxR], sRecvBase[kMaxR + 1];
  __shared__ int sRecvFirst[kMaxR], sRecvN[kMaxR];
  // replica list
  __shared__ int sRexp[kMaxL], sRrank[kMaxL], sRstart[kMaxL], sRcount[kMaxL], sRslot[kMaxL];
  // relay fallback: per-rank slot chains, and the regrouped list
  __shared__ int sHosted[kMaxR], sChainFirst[kMaxR], sChainLast[kMaxR], sChainNext[kMaxL];
  __shared__ int tExp[kMaxL], tRank[kMaxL], tCount[kMaxL], tSlot[kMaxL];
  __shared__ int sTmp[32];
  // bounded search: candidate order, copies left, per-rank out/took, generations, choices
  __shared__ int sCand[kMaxE], sCandG[kMaxE], sCap[kMaxE];
  __shared__ int sOut[kMaxR], sAvail[kMaxR], sPn[kMaxR], sPneed[kMaxR], sGs[kMaxR + 1], sCi[kMaxR];
  __shared__ int sNDonor, sNRecv, sMaxNeeded, sOverflow, sBad, sNOut, sRelayed, sDropped;
  __shared__ int sSteps, sFound;

  const int tid = threadIdx.x, nt = blockDim.x;
  const int E_loc = E / R;
  const int SK = S * K;
  const PlanLayout L(E, R, B);

  if (tid == 0) {
    sNDonor = 0;
    sNRecv = 0;
    sMaxNeeded = 0;
    sOverflow = 0;
    sBad = 0;
    sRelayed = 0;
    sDropped = 0;
    sSteps = 0;
    sFound = 0;
  }
  __syncthreads();
  // T_e and the bad-id flag
  for (int e = tid; e < E; e += nt) {
    int s = 0;
#pragma unroll 8
    for (int p = 0; p < R; ++p) s += counts[(size_t)p * E + e];
    sT[e] = s;
    sRepFirst[e] = 0;
    sRepN[e] = 0;
  }
  for (int p = tid; p < R; p += nt) {
    if (bad[p] != 0) atomicOr(&sBad, 1);
    sNP[p] = 0;
    sRecvFirst[p] = -1;
    sRecvN[p] = 0;
    sHosted[p] = 0;
    sChainFirst[p] = -1;
    sChainLast[p] = -1;
  }
  __syncthreads();
  // home loads and excess
  for (int r = tid; r < R; r += nt) {
    int l = 0;
    for (int e = r * E_loc; e < (r + 1) * E_loc; ++e) l += sT[e];
    sD[r] = l - SK;
  }
  __syncthreads();
  // donor order (d desc, r asc) and receiver order (-d desc, r asc) by counting ranks
  for (int r = tid; r < R; r += nt) {
    const int d = sD[r];
    sDonorPos[r] = -1;
    if (d > 0) {
      int pos = 0;
      for (int q = 0; q < R; ++q) {
        const int dq = sD[q];
        pos += (dq > d) || (dq == d && q < r);
      }
      sDonorPos[r] = pos;
      sDonorAt[pos] = r;
      atomicAdd(&sNDonor, 1);
    } else if (d < 0) {
      int pos = 0;
      for (int q = 0; q < R; ++q) {
        const int dq = sD[q];
        pos += (dq < d) || (dq == d && q < r);
      }
      sRecvAt[pos] = r;
      atomicAdd(&sNRecv, 1);
    }
  }
  __syncthreads();
  const int nDonor = sNDonor, nRecv = sNRecv;
  // pieces: rank of e inside its home group by (T desc, e asc), the load before
  // it in that order, and the piece it gives up
  for (int e = tid; e < E; e += nt) {
    const int r = e / E_loc, t = sT[e];
    int srank = 0, pre = 0;
    for (int f = r * E_loc; f < (r + 1) * E_loc; ++f) {
      const int tf = sT[f];
      if (tf > t || (tf == t && f < e)) {
        ++srank;
        pre += tf;
      }
    }
    const int d = sD[r];
    int a = 0;
    if (d > 0) a = min(t, max(0, d - pre));
    sSrank[e] = srank;
    sPre[e] = pre;
    sA[e] = a;
    sKeep[e] = t - a;
    if (a > 0) atomicAdd(&sNP[r], 1);
  }
  __syncthreads();
  // scans in donor order: piece index base and position in the donated-copy stream
  {
    int total;
    const int i = tid;
    const int r = (i < nDonor) ? sDonorAt[i] : 0;
    const int np = (i < nDonor) ? sNP[r] : 0;
    const int dd = (i < nDonor) ? sD[r] : 0;
    const int pbase = block_scan_excl(np, sTmp, &total);
    const int dbase = block_scan_excl(dd, sTmp, &total);
    if (i < nDonor) {
      sPieceBase0[i] = pbase;
      sDonorBase[i] = dbase;
    }
    // receiver stream positions
    const int q = (i < nRecv) ? sRecvAt[i] : 0;
    const int need = (i < nRecv) ? -sD[q] : 0;
    const int qbase = block_scan_excl(need, sTmp, &total);
    if (i < nRecv) sRecvBase[i] = qbase;
    if (i == 0) sRecvBase[nRecv] = total;
  }
  __syncthreads();
  const int qTot = sRecvBase[nRecv];
  // each piece: its place in the piece order, stream start, receivers it spans
  for (int e = tid; e < E; e += nt) {
    const int a = sA[e];
    if (a == 0) continue;
    const int r = e / E_loc;
    const int dpos = sDonorPos[r];
    const int pidx = sPieceBase0[dpos] + sSrank[e];
    const int P = sDonorBase[dpos] + sPre[e];
    const int hiPos = min(P + a, qTot);
    int jlo = 0, cnt = 0;
    if (P < hiPos) {
      // last receiver j with start <= x: binary search over sRecvBase[0..nRecv)
      int lo = 0, hi = nRecv;  // invariant: answer in [lo, hi)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sRecvBase[mid] <= P) lo = mid; else hi = mid;
      }
      jlo = lo;
      lo = jlo;
      hi = nRecv;
      const int last = hiPos - 1;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sRecvBase[mid] <= last) lo = mid; else hi = mid;
      }
      cnt = lo - jlo + 1;
    }
    sPieceE[pidx] = e;
    sPieceP[pidx] = P;
    sPieceJlo[pidx] = jlo;
    sPieceCnt[pidx] = cnt;
  }
  __syncthreads();
  int nPieces;
  {
    int total;
    // number of pieces = sum over donors
    const int v = (tid < nDonor) ? sNP[sDonorAt[tid]] : 0;
    block_scan_excl(v, sTmp, &total);
    nPieces = total;
  }
  int nRep;
  {
    int total;
    const int v = (tid < nPieces) ? sPieceCnt[tid] : 0;
    const int base = block_scan_excl(v, sTmp, &total);
    nRep = total;
    if (tid < nPieces) {
      const int e = sPieceE[tid], P = sPieceP[tid], a = sA[e], jlo = sPieceJlo[tid];
      const int cnt = sPieceCnt[tid];
      if (cnt > 0) {
        sRepFirst[e] = base;
        sRepN[e] = cnt;
      }
      for (int u = 0; u < cnt; ++u) {
        const int j = jlo + u;
        const int lo = max(P, sRecvBase[j]);
        const int hi = min(P + a, sRecvBase[j + 1]);
        const int m = base + u;
        sRexp[m] = e;
        sRrank[m] = sRecvAt[j];
        sRstart[m] = sKeep[e] + (lo - P);
        sRcount[m] = hi - lo;
      }
    }
  }
  __syncthreads();
  // slots: a receiver's replicas are consecutive in emission order
  for (int m = tid; m < nRep; m += nt) {
    const int q = sRrank[m];
    int s = m;
    while (s > 0 && sRrank[s - 1] == q) --s;
    const int slot = m - s;
    sRslot[m] = slot < B ? slot : -1;
    if (slot >= B) atomicOr(&sOverflow, 1);
    if (m == s) sRecvFirst[q] = m;
    if (m == nRep - 1 || sRrank[m + 1] != q) {
      sRecvN[q] = slot + 1;
      atomicMax(&sMaxNeeded, slot + 1);
    }
  }
  __syncthreads();
  int nOut = nRep;
  if (sOverflow) {  // uniform: the walk does not fit in B slots somewhere
    if (tid == 0) {
      RelayState st{sRexp, sRrank, sRcount, sRslot, sKeep, sHosted, sChainFirst, sChainLast,
                    sChainNext, E_loc, B, 0};
      int nd = 0;
      sRelayed = relay_pass(st, nRep, &nd);
      sDropped = nd;
      sNOut = st.w;
    }
    __syncthreads();
    if (sDropped && B >= 1) {  // uniform: the bounded search
      // candidate order (homes by (d desc, r asc), experts by (T desc, e asc) = sSrank),
      // copies left, and generation 0 (the receivers in their walk order)
      for (int e = tid; e < E; e += nt) {
        const int r = e / E_loc, d = sD[r];
        int pos = 0;
        for (int q = 0; q < R; ++q) {
          const int dq = sD[q];
          pos += (dq > d) || (dq == d && q < r);
        }
        sCand[pos * E_loc + sSrank[e]] = e;
        sCandG[pos * E_loc + sSrank[e]] = r;
        sCap[e] = sT[e];
      }
      for (int r = tid; r < R; r += nt) {
        sOut[r] = 0;
        sAvail[r] = sD[r] < 0 ? kTaken : sD[r];
      }
      for (int j = tid; j < nRecv; j += nt) {
        sPn[j] = sRecvAt[j];
        sPneed[j] = -sD[sRecvAt[j]];
      }
      if (tid == 0) {
        sGs[0] = 0;
        sGs[1] = nRecv;
      }
      __syncthreads();
      if (tid < 64) {
        const SearchState ss{sCand, sCandG, sCap, sOut, sAvail, sPn, sPneed, sGs, sCi, sD, E, R};
        int steps = 0;
        const int n = relay_search(ss, nRecv, tid, &steps);
        if (tid == 0) {
          sSteps = steps;
          sFound = n >= 0;
          if (n >= 0) {
            sNOut = n;
            sDropped = 0;
          }
        }
      }
      __syncthreads();
      if (sFound) {  // uniform: the search's plan replaces the relay pass's
        for (int m = tid; m < sNOut; m += nt) {
          const int c = sCi[m];
          sRexp[m] = sCand[c < E ? c : c - E];
          sRrank[m] = sPn[m];
          sRcount[m] = sPneed[m];
          sRslot[m] = 0;
        }
        for (int e = tid; e < E; e += nt) sKeep[e] = sCap[e];
        for (int r = tid; r < R; r += nt) sHosted[r] = 0;
        __syncthreads();
        for (int m = tid; m < sNOut; m += nt) sHosted[sPn[m]] = 1;
      }
      __syncthreads();
    }
    // sSrank (per expert) is free now: first list index of each expert
    for (int e = tid; e < E; e += nt) {
      sSrank[e] = 0x7fffffff;
      sRepFirst[e] = 0;
      sRepN[e] = 0;
    }
    __syncthreads();
    nOut = sNOut;
    for (int m = tid; m < nOut; m += nt) atomicMin(&sSrank[sRexp[m]], m);
    __syncthreads();
    // gather each expert's entries: experts by first entry, entries in pass order
    for (int m = tid; m < nOut; m += nt) {
      const int e = sRexp[m], fi = sSrank[e];
      int pos = 0;
      for (int k = 0; k < nOut; ++k) {
        const int ek = sRexp[k];
        pos += (sSrank[ek] < fi) || (ek == e && k < m);
      }
      tExp[pos] = e;
      tRank[pos] = sRrank[m];
      tCount[pos] = sRcount[m];
      tSlot[pos] = sRslot[m];
    }
    __syncthreads();
    for (int m = tid; m < nOut; m += nt) {
      sRexp[m] = tExp[m];
      sRrank[m] = tRank[m];
      sRcount[m] = tCount[m];
      sRslot[m] = tSlot[m];
    }
    __syncthreads();
    // tile each expert's copies: home first, then its entries in order
    for (int m = tid; m < nOut; m += nt) {
      const int e = sRexp[m];
      int st = sKeep[e], k = m - 1;
      for (; k >= 0 && sRexp[k] == e; --k) st += sRcount[k];
      sRstart[m] = st;
      if (k == m - 1) {
        int n = 1;
        while (m + n < nOut && sRexp[m + n] == e) ++n;
        sRepFirst[e] = m;
        sRepN[e] = n;
      }
    }
  } else {
    for (int q = tid; q < R; q += nt) sHosted[q] = sRecvN[q];
  }
  __syncthreads();
  // write the blob, each word exactly once
  const int status = (sBad ? MOE_DEV_BAD_EXPERT_ID : 0) | (sDropped ? MOE_DEV_SLOT_OVERFLOW : 0);
  if (tid == 0) {
    plan[0] = status;
    plan[1] = nOut;
    plan[2] = sMaxNeeded;
    plan[3] = nDonor;
    plan[4] = nRecv;
    plan[5] = nPieces;
    plan[6] = sRelayed;
    plan[7] = sSteps;
    if (dev_status) *dev_status = (uint32_t)status;
  }
  for (int e = tid; e < E; e += nt) {
    plan[L.off_T + e] = sT[e];
    plan[L.off_keep + e] = sKeep[e];
    plan[L.off_rep_first + e] = sRepFirst[e];
    plan[L.off_rep_n + e] = sRepN[e];
  }
  for (int m = tid; m < E + R; m += nt) {
    const bool used = m < nOut;
    plan[L.off_rexp + m] = used ? sRexp[m] : -1;
    plan[L.off_rrank + m] = used ? sRrank[m] : -1;
    plan[L.off_rslot + m] = used ? sRslot[m] : -1;
    plan[L.off_rstart + m] = used ? sRstart[m] : 0;
    plan[L.off_rcount + m] = used ? sRcount[m] : 0;
  }
  // slot tables: slots 0..hosted-1 of a rank are written by their entries,
  // the rest are empty
  for (int m = tid; m < nOut; m += nt) {
    const int j = sRslot[m];
    if (j < 0) continue;
    const int w = sRrank[m] * B + j;
    plan[L.off_sexp + w] = sRexp[m];
    plan[L.off_sstart + w] = sRstart[m];
    plan[L.off_scount + w] = sRcount[m];
  }
  for (int w = tid; w < R * B; w += nt) {
    if (w % B < sHosted[w / B]) continue;
    plan[L.off_sexp + w] = -1;
    plan[L.off_sstart + w] = 0;
    plan[L.off_scount + w] = 0;
  }
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_plan_words(const moe_dims *d) {
  if (!dims_ok(d)) return 0;
  return (size_t)PlanLayout(d->E, d->R, d->B).words;
}

extern "C" size_t moe_plan_workspace_bytes(const moe_dims *d) {
  if (!dims_ok(d)) return 0;
  const int nchunk = ceil_div((long long)d->S * d->K, kPlanChunk);
  return (size_t)d->R * nchunk * (d->E + 1) * sizeof(int32_t) + (size_t)d->R * sizeof(int32_t);
}

// The three launches of a plan, with scratch `ws` of at least moe_plan_workspace_bytes(d)
// bytes: per-chunk histograms, then the per-rank bad-id counts.  Every scratch word is written
// before it is read, so the scratch needs no clearing.
static moe_status_t plan_launch(const moe_dims *d, const int32_t *topk_idx, int32_t *counts,
                                int32_t *plan, uint32_t *dev_status, void *ws,
                                hipStream_t stream) {
  const int SK = d->S * d->K;
  const int nchunk = ceil_div(SK, kPlanChunk);
  int32_t *partial = (int32_t *)ws;
  int32_t *bad = partial + (size_t)d->R * nchunk * (d->E + 1);
  hipLaunchKernelGGL(k_plan_hist, dim3(nchunk, d->R), dim3(kHistThreads), 0, stream, topk_idx,
                     partial, SK, d->E, nchunk);
  hipLaunchKernelGGL(k_plan_reduce, dim3(d->R), dim3(kHistThreads), 0, stream, partial, counts,
                     bad, d->E, nchunk);
  hipLaunchKernelGGL(k_plan_solve, dim3(1), dim3(kSolveThreads), 0, stream, counts, bad, plan,
                     dev_status, d->R, d->S, d->K, d->E, d->B);
  return launch_status();
}

extern "C" moe_status_t moe_plan(const moe_dims *d, const int32_t *topk_idx, int32_t *counts,
                                 int32_t *plan, uint32_t *dev_status, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
  if (!dims_ok(d) || !topk_idx || !counts || !plan || !ws) return MOE_EINVAL;
  if (ws_bytes < moe_plan_workspace_bytes(d)) return MOE_ENOSPACE;
  return plan_launch(d, topk_idx, counts, plan, dev_status, ws, stream);
}

// ---- moe_plan_noalloc: the same plan with its scratch in a static device array ----------
// For callers that cannot allocate (HIP graph capture, serving loops).  The array is a
// file-scope __device__ object, so every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code the array's name is only a host-side
// stand-in for the symbol: its device address is looked up once per device with
// hipGetSymbolAddress (on the entry point's first call with that device current) and that
// address, never the name, is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[MOE_PLAN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void *g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
}  // namespace

// Device address of the current device's copy of `scratch`, or nullptr.
static void *plan_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev]() {
    void *ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

extern "C" moe_status_t moe_plan_noalloc(const moe_dims *d, const int32_t *topk_idx,
                                         int32_t *counts, int32_t *plan, uint32_t *dev_status,
                                         hipStream_t stream) {
  if (!dims_ok(d) || !topk_idx || !counts || !plan) return MOE_EINVAL;
  if (moe_plan_workspace_bytes(d) > MOE_PLAN_NOALLOC_SCRATCH_BYTES) return MOE_ENOSPACE;
  void *ws = plan_scratch();
  if (!ws) return MOE_EHIP;
  return plan_launch(d, topk_idx, counts, plan, dev_status, ws, stream);
}
