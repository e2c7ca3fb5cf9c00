// moe_group_gemm: grouped GEMM over one contiguous [G, Kd, N] weight tensor,
// groups addressed purely by row index, segments given by cu_seqlens.
//
// Pages: ainovat.com "Moonshot AI Open-Sources MoonEP", contract paragraph
// (the group GEMM consumes a single [E+B, H, H'] weight tensor and the
// planner's cu_seqlens selects the active rows) and contiguity paragraph
// (experts are addressed by row index, so the tensor must be contiguous).
//
// bf16 path (MFMA, gfx950):
//   * persistent grid of one workgroup per CU; every workgroup rebuilds the
//     tile table from cu_seqlens in LDS (no host sync, the grid is sized from
//     the machine, not from the routing);
//   * 256x256 output tile, K step 32 (DGRAD: 64-wide stages, see tile_mma64),
//     v_mfma_f32_32x32x16_bf16 blocks with fp32 accumulators; FWD and DGRAD
//     run 4 waves (one per SIMD) of 128x128, WGRAD and the gated FWD 8 waves
//     of 128x64;
//   * operands go global -> LDS with direct-to-LDS buffer loads (no register
//     staging) into a 4-stage ring, XOR-swizzled by 16-byte chunks so the
//     fragment reads are conflict-free; an operand whose contraction index is
//     contiguous is read with ds_read_b128, one whose contraction index is
//     strided (the weight in FWD, both operands in WGRAD) with the
//     transposing ds_read_b64_tr_b16;
//   * interleaved K loop: each wave issues one fragment read or load behind
//     each MFMA, and the per-step scalar work is kept small enough to fit the
//     issue cycles an MFMA leaves (see tile_mma; the 8-wave loop runs
//     unrolled over the ring's stages);
//   * the MFMA is issued as (column-side x row-side) so each lane ends with
//     4 consecutive output columns; output tiles leave through LDS so that
//     global memory sees whole rows (bf16 stores; WGRAD's fp32
//     read-modify-write, see wgrad_rmw);
//   * blockIdx is remapped so the 32 workgroups of one XCD work on
//     neighbouring tiles (shared weight and activation panels in that XCD's
//     L2); tiles are walked in groups of 8 row-tiles;
//   * with a workspace, the row-operand GEMMs split the contraction of the
//     tiles of a partial last round over all workgroups and add the parts in
//     a second kernel (see sk_plan);
//   * WGRAD tiles cost their segment's row count: segments are dealt longest
//     first and rounds of tiles alternate direction (see order_by_length).
// fp32 path: plain vector-ALU kernels (small shapes only).
#include "common.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kMaxDim = 1 << 22;  // largest Kd and N (per-lane load offsets stay in 32 bits)
constexpr int kMaxG = 1088;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

// Wave layouts of the 256x256 output tile (2 waves along rows, WN along columns).
//   Waves<2>: 4 waves, one per SIMD, each 128 x 128 = 4 x 4 blocks of 32x32 (fp32
//             accumulators in the accumulation registers); FWD and DGRAD.
//   Waves<4>: 8 waves, two per SIMD, each 128 x 64 = 4 x 2 blocks; WGRAD and the gated FWD,
//             whose epilogues need the registers the larger wave tile takes.
template <int WN>
struct Waves {
  static constexpr int M = 2, N = WN, n = M * N, threads = 64 * n;
  static constexpr int TM = BM / (32 * M), TN = BN / (32 * N);
  static constexpr int blk = 16 / n;    // 1-KB blocks per wave per operand per K step
  static constexpr int loads = 2 * blk; // direct-to-LDS loads per wave per K step
};
constexpr int kMaxBlk = 4;

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes) {
  const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
constexpr int kOOB = 0x7FFFFFF0;  // an offset past every resource: the load returns zero

typedef __attribute__((address_space(3))) void *lds_vptr;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) bf16x4_t *lds_bf16x4_ptr;

// LDS ring: kStages K-steps of BK=32; each stage holds the row-side operand then the
// column-side operand, 256 x 32 bf16 = 16 KB each, no padding (bank spreading is done by
// an XOR swizzle of 16-byte chunks, applied on the global side of the direct-to-LDS loads).
constexpr int kStages = 4;
constexpr int OP_ELEMS = 256 * BK;            // one operand of one stage
constexpr int STAGE_ELEMS = 2 * OP_ELEMS;

// Direct-to-LDS loads of one operand tile (256 rows x BK contraction per K step).  Each
// wave instruction writes 64 lanes x 16 B = 1 KB of LDS contiguously; the 16 blocks of an
// operand tile are shared out over the waves.
//  contiguous source (row r, contraction c at base[r*ld + c]): LDS is [256][BK], 64 B per row;
//    16-byte chunk k of row r sits at position k ^ ((r >> 2) & 3);
//  strided source (row r, contraction c at base[c*ld + r]): LDS is [BK][256], 512 B per
//    contraction row; chunk k (rows 8k..8k+7) of contraction row c sits at k ^ (4 * (c & 3)).
// The per-lane byte offset of each block is fixed for the tile (rows past the tile get an
// offset past every buffer, so they load zeros); a K step only moves the buffer resource:
// its base advances by one step and its byte count shrinks by the same amount, so the
// hardware range check still zero-fills contraction rows past the end of a strided operand,
// and a step past the last gets a zero-byte resource.  A contiguous operand whose
// contraction length is not a multiple of BK also needs a per-lane column test in its last
// step (RAGGED).
struct DmaOp {
  const char *base;  // byte address of element (row 0, contraction 0) of the tile
  long long bytes;   // bytes readable from base
  long long step;    // bytes per K step
  int voff[kMaxBlk]; // per-lane byte offset of this wave's blocks, or kOOB
  int kc[kMaxBlk];   // contraction index of each block's chunk within a K step
};

template <class W, bool CONTIG>
__device__ inline void dma_init(DmaOp &d, const uint16_t *base, long long bytes, int ld,
                                int row_lim) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  d.base = (const char *)base;
  d.bytes = bytes;
  d.step = CONTIG ? BK * 2 : (long long)BK * ld * 2;
#pragma unroll
  for (int u = 0; u < W::blk; ++u) {
    const int blk = u * W::n + wid;                // 1-KB block of the 16-KB tile
    const int o = blk * 1024 + lane * 16;          // this lane's LDS byte offset
    if (CONTIG) {
      const int r = o >> 6, p = (o >> 4) & 3;
      const int k = p ^ ((r >> 2) & 3);
      d.voff[u] = r < row_lim ? (r * ld + k * 8) * 2 : kOOB;
      d.kc[u] = k * 8;
    } else {
      const int cr = o >> 9, p = (o >> 4) & 31;
      const int k = p ^ (4 * (cr & 3));
      d.voff[u] = k * 8 < row_lim ? (cr * ld + k * 8) * 2 : kOOB;
      d.kc[u] = cr;
    }
  }
}

// Byte count of an operand's buffer resource at K step kt: the bytes left from the step's
// base, clamped to [0, kOOB], and 0 past the last step.  Worked out once per tile so that a K
// step costs a few 32-bit scalar operations (the step's instructions share one wave's issue
// slots with its MFMAs): the first `ksat` steps have more than kOOB bytes left; from then on
// the count fits 31 bits and equals the low word of the byte count minus kt steps, in 32-bit
// arithmetic (it never falls below -2^31: a tile ends within a step of its operand's end).
struct DmaCount {
  uint32_t lo;  // low 32 bits of the byte count at step 0
  int ksat;     // steps whose count saturates at kOOB
};

__device__ inline DmaCount dma_count(long long bytes, long long step) {
  DmaCount c;
  c.lo = (uint32_t)bytes;
  c.ksat = 0;
  if (bytes >= kOOB) {
    // operands over 2 GB only; the empty asm keeps the division's set-up from being hoisted
    // out of the tile loop (where its registers would stay live for nothing)
    asm volatile("" : "+s"(step));
    c.ksat = (int)((bytes - kOOB) / step) + 1;
  }
  // the division may run on the vector unit; the count is wave-uniform and must stay in
  // scalar registers (it becomes part of a buffer resource)
  c.ksat = __builtin_amdgcn_readfirstlane(c.ksat);
  return c;
}

__device__ inline int dma_bytes_at(const DmaCount &c, int step, int kt, int nk) {
  int n = (int)(c.lo - (uint32_t)kt * (uint32_t)step);
  n = n < 0 ? 0 : n;
  n = kt < c.ksat ? kOOB : n;
  return kt < nk ? n : 0;
}

// Buffer resource of K step kt of an operand (a zero-byte resource past the last step).
__device__ inline __amdgpu_buffer_rsrc_t dma_rsrc(const DmaOp &d, const DmaCount &c, int kt,
                                                  int nk) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(d.base + (long long)kt * d.step),
                                           (short)0, dma_bytes_at(c, (int)d.step, kt, nk),
                                           0x00020000);
}

// This wave's load u of K step kt into the operand's LDS region at byte address `lds_op`
// (+ this wave's block offset `wave_off`).
template <class W, bool CONTIG, bool RAGGED>
__device__ inline void dma_one(const DmaOp &d, __amdgpu_buffer_rsrc_t rs, uint32_t lds_op,
                               uint32_t wave_off, int kt, int c_lim, int u) {
  int off = d.voff[u];
  if (CONTIG && RAGGED) off = kt * BK + d.kc[u] < c_lim ? off : kOOB;
  // buffer_load_dwordx4 ... lds: 16 bytes per lane straight into LDS at M0 + 16 * lane.
  // Written as asm so the compiler does not track it: its alias analysis cannot tell the
  // ring's stages apart and would drain every load at each barrier.  The load has no
  // register result (nothing in flight can overwrite a VGPR); the "memory" clobber keeps
  // LDS accesses on their side of it; completion is ordered only by the explicit vmcnt
  // waits and barriers of the K loop.  M0 is set by the compiler from the "{m0}" operand;
  // the asm starts with one wait state, because on this architecture family an LDS-DMA
  // load must not read M0 in the cycle after a scalar write to it (the compiler pads its
  // own LDS-DMA loads the same way).
  const uint32_t m0 = lds_op + wave_off + u * W::n * 1024;
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off),
      "s"(rs), "{m0}"(m0)
      : "memory");
}

// MFMA operand t of lane `lane` (rows wbase + 32t .. +31 for a contiguous operand) at
// contraction 16*ks + 8*(lane/32) .. +8.
template <bool CONTIG>
__device__ inline bf16x8 read_operand(const uint16_t *src, int wbase, int t, int lane, int ks) {
  if (CONTIG) {
    const int r = wbase + 32 * t + (lane & 31);
    const int k = 2 * ks + (lane >> 5);
    const int p = k ^ ((r >> 2) & 3);
    return __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + r * BK + p * 8));
  } else {
    // Two transposing reads of 4 contraction values each.  Lane rule of
    // ds_read_b64_tr_b16 (per 16-lane group): lane a = 4u+q supplies the address of 4
    // consecutive row values at contraction c0+u, rows r0+4q..+3; lane j of the group then
    // receives row r0+j at contraction c0..c0+3.  The stored 16-byte chunk of rows r..r+7
    // at contraction c sits at position (r>>3) ^ 4(c&3), and c&3 == u here, so the
    // address depends on (t, lane) only; sub-step and half are immediate offsets.
    const int g = lane >> 4, a = lane & 15;
    const int u = a >> 2, q = a & 3;
    const int r = wbase + 32 * t + 16 * (g & 1) + 4 * q;
    const int c = ks * 16 + 8 * (g >> 1) + u;
    const uint16_t *p0 = src + c * 256 + ((r >> 3) ^ (4 * u)) * 8 + (r & 7);
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)p0);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p0 + 4 * 256));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// ---- Gathered row operand ------------------------------------------------------------
// With a gather, row m of the row operand is token row idx[m] / div of x: the row is read
// straight from the token rows as the operand is loaded, so the tokens need not be permuted
// into expert-grouped order first.  Token rows are scattered over x, which may be larger than
// a buffer resource's 32-bit offsets reach, so these loads take per-lane 64-bit addresses
// (global_load_lds_dwordx4: 16 bytes per lane into LDS at M0 + 16 * lane, the same layout as
// the buffer form).  A chunk outside the operand (contraction past its end, rows past a
// segment, columns past the output) reads from g_zeros instead, the gathered form of the
// buffer resource's zero fill.
struct GatherParams {
  const char *x;       // token rows
  uint32_t ld_bytes;   // bytes per token row (the operand's contraction or row length * 2)
  const int32_t *idx;  // gather entry of every operand row
  int n_tok;           // token rows in x
  uint32_t magic;      // floor(e / div) = mulhi(2 e, magic) >> shift for 0 <= e < 2^31
  int shift;
  int div;
};

// 512 zero bytes: a __device__ object, zero-initialised when the code object loads and never
// written.
__device__ __align__(256) uint16_t g_zeros[256];

__device__ inline int gather_div(int e, const GatherParams &gp) {
  return (int)(__umulhi((uint32_t)e << 1, gp.magic) >> gp.shift);
}

// Token row of gather entry e, or -1 when e does not name one of the n_tok rows.
__device__ inline int gather_token(int e, const GatherParams &gp) {
  const int t = gather_div(e, gp);
  return (e >= 0 && t < gp.n_tok) ? t : -1;
}

// A load of one 16-byte chunk per lane into LDS at M0 + 16 * lane from a 64-bit address.
// As dma_one: asm so the compiler does not track it (ordering is by the explicit vmcnt waits),
// no register result, one wait state after the M0 write.
__device__ inline void gload_lds(const char *p, uint32_t m0) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off" ::"v"(p),
      "{m0}"(m0)
      : "memory");
}

// A 32-bit load from a wave-uniform address, through the scalar data cache (SMEM, counted
// by lgkmcnt): it leaves the vector-memory counter, which orders the operand loads, alone.
__device__ inline int load_uniform(const int32_t *p) {
  typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;
  return *(const_i32_ptr)p;
}

// Gathered operand whose contraction index is contiguous (the activation rows of FWD): each
// lane loads one 16-byte chunk of one row per block and K step; its row is fixed for the
// tile, so the token of each block's row is looked up once per tile.
struct GatherC {
  const char *x;
  uint32_t ld_bytes;
  int tok[kMaxBlk];  // token row of this lane's row in each block (0 for rows past the tile)
  int coff;          // byte offset of this lane's chunk in the row at K step 0 of the tile
  int zc;            // byte offset of this lane's chunk in g_zeros
  int kc;            // contraction index of this lane's chunk within a K step
};

// Row r of block blk of a contiguous [256][BK] operand tile is 16 blk + lane / 4 and its chunk
// is (lane & 3) ^ ((r >> 2) & 3) = (lane & 3) ^ ((lane >> 4) & 3) (see dma_init).
template <class W>
__device__ inline void gather_c_init(GatherC &g, const GatherParams &gp, int m0, int rows,
                                     int k0) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int k = (lane & 3) ^ ((lane >> 4) & 3);
  g.x = gp.x;
  g.ld_bytes = gp.ld_bytes;
  g.kc = k * 8;
  g.zc = k * 16;
  g.coff = k * 16 + k0 * (BK * 2);
#pragma unroll
  for (int u = 0; u < W::blk; ++u) {
    const int r = (u * W::n + wid) * 16 + (lane >> 2);
    int tok = 0;
    if (r < rows) tok = max(gather_token(gp.idx[m0 + r], gp), 0);
    g.tok[u] = tok;
  }
}

// Load u of K step kt (contraction kt * BK .. of the tile's part); chunks at or past c_lim
// (a ragged last step, or a step past the last) read zeros.
template <class W>
__device__ inline void gather_c_one(const GatherC &g, uint32_t lds_op, uint32_t wave_off, int kt,
                                    int c_lim, int u) {
  const char *p = g.x + (unsigned long long)(uint32_t)g.tok[u] * g.ld_bytes + g.coff +
                  (long long)kt * (BK * 2);
  if (kt * BK + g.kc >= c_lim) p = (const char *)g_zeros + g.zc;
  gload_lds(p, lds_op + wave_off + u * W::n * 1024);
}

// Gathered operand whose contraction index is strided (the activation rows of WGRAD, where
// the contraction runs over the segment's rows): each block of a K step covers two
// contraction rows (lanes 0-31 and 32-63), so the rows, and their tokens, change every step.
// Their gather entries are read with scalar loads (gather_s_fetch) right after a mid-step
// barrier; each lane then works out its own row's token and address with vector arithmetic
// (gather_s_addr_part, two parts pinned to two MFMA slots): block 0's in the last two slots
// of the same half step, block 1's in the next half step's first slots, ahead of its load.
// Scalar loads share the LDS reads' counter and return out of order, so any wait while one is
// outstanding must wait for everything: issued where the counter has just been drained and
// consumed after the half step's last fragment read, they cost neither an early wait for the
// fragments nor arithmetic ahead of a step's first MFMA.
struct GatherS {
  GatherParams gp;
  const int32_t *idx_seg;  // gather entries of the segment's rows (wave-uniform)
  int row_w;         // 2 * wave index: this wave's first row of a K step's block
  int m0, len;       // first operand row and row count of the segment (wave-uniform)
  uint32_t e_lim;    // gather entries in [0, e_lim) name a token row
  const char *xcol;  // x + this lane's column byte offset
  long long ozero;   // xcol + ozero = this lane's chunk of g_zeros (wave-uniform)
  int half;          // which of a block's two contraction rows this lane loads
  int e[kMaxBlk][2];          // gather entries of the rows of the next step to be issued
  const char *addr[kMaxBlk];  // this lane's load addresses for the step being issued
  int tok[kMaxBlk], ok[kMaxBlk];  // between the two parts of gather_s_addr_part
};

// Block blk = u n + wid of a strided [BK][256] operand tile covers contraction rows 2 blk and
// 2 blk + 1; lane chunk p = lane & 31 of its row sits at column chunk p ^ (4 (cr & 3)) with
// cr & 3 = 2 (wid & 1) + lane / 32 (see dma_init).  A chunk at or past the operand's last
// column is moved onto its last chunk: its values only reach output rows past the edge, which
// are never stored.
template <class W>
__device__ inline void gather_s_init(GatherS &g, const GatherParams &gp, int m0, int len, int i0,
                                     int Kd) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int k = (lane & 31) ^ (4 * (2 * (wid & 1) + (lane >> 5)));
  const int col = min(i0 + k * 8, Kd - 8);
  g.gp = gp;
  g.m0 = __builtin_amdgcn_readfirstlane(m0);
  g.len = __builtin_amdgcn_readfirstlane(len);
  g.idx_seg = gp.idx + g.m0;
  g.row_w = __builtin_amdgcn_readfirstlane(2 * wid);
  const unsigned long long lim = (unsigned long long)gp.n_tok * gp.div;
  g.e_lim = lim < 0x80000000ull ? (uint32_t)lim : 0x80000000u;
  g.xcol = gp.x + (long long)col * 2;
  g.ozero = (long long)((uintptr_t)g_zeros - (uintptr_t)gp.x) - (long long)i0 * 2;
  g.half = lane >> 5;
}

// First segment row of block u's pair of contraction rows in K step kt (wave-uniform).
template <class W>
__device__ inline int gather_s_row(const GatherS &g, int kt, int u) {
  return kt * BK + 2 * u * W::n + g.row_w;
}

// Scalar loads of the gather entries of K step kt's rows (rows past the segment read its
// last row's entry, which gather_s_addr then ignores).
template <class W>
__device__ inline void gather_s_fetch(GatherS &g, int kt) {
#pragma unroll
  for (int u = 0; u < W::blk; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      g.e[u][h] = load_uniform((const int32_t *)((const char *)g.idx_seg +
                                                 (uint32_t)min(gather_s_row<W>(g, kt, u) + h,
                                                               g.len - 1) * 4u));
}

// This lane's address for load u of K step kt, from the entries gather_s_fetch(kt) read, in
// two parts so that each fits beside one MFMA: the lane's token and whether its row is real
// (part 0: a row past the segment, or an entry that names no token row, reads g_zeros, as
// the permute writes zeros for such rows), then the address (part 1).  The empty asms pin
// each part's arithmetic to its call site: left alone, the compiler gathers it ahead of a
// step's first MFMAs.
template <class W>
__device__ inline void gather_s_addr_part(GatherS &g, int kt, int u, int part) {
  if (part == 0) {
    int e0 = g.e[u][0], e1 = g.e[u][1];
    asm volatile("" : "+s"(e0), "+s"(e1));
    const int e = g.half ? e1 : e0;
    int tok = (int)(__umulhi((uint32_t)e << 1, g.gp.magic) >> g.gp.shift);
    int ok = (uint32_t)e < g.e_lim && gather_s_row<W>(g, kt, u) + g.half < g.len;
    asm volatile("" : "+v"(tok), "+v"(ok));
    g.tok[u] = tok;
    g.ok[u] = ok;
  } else {
    int tok = g.tok[u], ok = g.ok[u];
    asm volatile("" : "+v"(tok), "+v"(ok));
    const char *p = g.xcol + (unsigned long long)(uint32_t)tok * g.gp.ld_bytes;
    g.addr[u] = ok ? p : g.xcol + g.ozero;
  }
}

template <class W>
__device__ inline void gather_s_addr(GatherS &g, int kt, int u) {
  gather_s_addr_part<W>(g, kt, u, 0);
  gather_s_addr_part<W>(g, kt, u, 1);
}

template <class W>
__device__ inline void gather_s_addr(GatherS &g, int kt) {
#pragma unroll
  for (int u = 0; u < W::blk; ++u) gather_s_addr<W>(g, kt, u);
}

template <class W>
__device__ inline void gather_s_one(const GatherS &g, uint32_t lds_op, uint32_t wave_off, int u) {
  gload_lds(g.addr[u], lds_op + wave_off + u * W::n * 1024);
}

template <int N>
__device__ inline void waitcnt_vm() {
  // s_waitcnt vmcnt(N), expcnt and lgkmcnt at their maximum (no wait on them);
  // vmcnt bits [3:0] low, [15:14] high
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One contraction sub-step (16) of this wave's MFMA operands.
template <class W>
struct Frags {
  bf16x8 a[W::TM], b[W::TN];
};

template <class W, bool A_CONTIG, bool B_CONTIG>
__device__ inline void read_frags(Frags<W> &f, const uint16_t *stage, int wi, int wj, int lane,
                                  int ks) {
#pragma unroll
  for (int t = 0; t < W::TM; ++t) f.a[t] = read_operand<A_CONTIG>(stage, wi, t, lane, ks);
#pragma unroll
  for (int t = 0; t < W::TN; ++t)
    f.b[t] = read_operand<B_CONTIG>(stage + OP_ELEMS, wj, t, lane, ks);
}

struct TileArgs {
  DmaOp a, b;
  DmaCount ca, cb;    // byte counts of a and b (tile_mma works them out)
  int c_len, nk;
  uint32_t wave_off;  // this wave's 1-KB block offset within an operand tile (wave-uniform)
  GatherC gc;         // the row-side operand gathered from token rows (AG == 1)
  GatherS gs;         // (AG == 2)
};

// Row-side operand source of the K loop: AG = 0 buffer loads from one operand tensor;
// AG = 1 gathered, contraction contiguous (FWD); AG = 2 gathered, contraction strided (WGRAD).
// This wave's loads of K step kt (both operands) into LDS stage `stage`; with AG == 2,
// gs.addr must hold the addresses of step kt (gather_s_addr).
template <class W, bool A_CONTIG, bool B_CONTIG, bool RAGGED, int AG>
__device__ inline void dma_step(const uint16_t *lds, int stage, const TileArgs &ta,
                                const GatherS &gs, int kt) {
  const uint32_t st = (uint32_t)(uintptr_t)(lds_vptr)(lds + stage * STAGE_ELEMS);
  const __amdgpu_buffer_rsrc_t rb = dma_rsrc(ta.b, ta.cb, kt, ta.nk);
  if constexpr (AG == 0) {
    const __amdgpu_buffer_rsrc_t ra = dma_rsrc(ta.a, ta.ca, kt, ta.nk);
#pragma unroll
    for (int u = 0; u < W::blk; ++u)
      dma_one<W, A_CONTIG, RAGGED>(ta.a, ra, st, ta.wave_off, kt, ta.c_len, u);
  } else if constexpr (AG == 1) {
#pragma unroll
    for (int u = 0; u < W::blk; ++u) gather_c_one<W>(ta.gc, st, ta.wave_off, kt, ta.c_len, u);
  } else {
#pragma unroll
    for (int u = 0; u < W::blk; ++u) gather_s_one<W>(gs, st, ta.wave_off, u);
  }
#pragma unroll
  for (int u = 0; u < W::blk; ++u)
    dma_one<W, B_CONTIG, RAGGED>(ta.b, rb, st + OP_ELEMS * 2, ta.wave_off, kt, ta.c_len, u);
}

// One 256x256 output tile: out_tile[i][j] = sum_c Aop(i, c) * Bop(j, c), BK = 32 per K
// step, K step k in LDS stage k % 4.
//
// A K step is two half steps, one per contraction sub-step of 16, each of TM*TN MFMAs;
// behind each MFMA the wave issues at most one memory operation for later, so the matrix
// unit is fed while reads and loads are in flight:
//   half A of step k: MFMAs on sub-step 0 (registers F0); reads sub-step 1 of step k into
//                     F1; issues its loads of the row-side operand of step k+3 into stage
//                     (k+3) % 4;
//   wait until at most the loads of step k+2 and the row-side loads of step k+3 are in
//   flight (so step k+1 has landed), barrier;
//   half B of step k: MFMAs on sub-step 1 (F1); reads sub-step 0 of step k+1 into F0;
//                     issues its loads of the column-side operand of step k+3.
// Stage (k+3) % 4 last held step k-1, whose reads every wave finished before the barrier in
// the middle of step k-1 (the barrier waits for this wave's LDS reads), and the barrier in
// the middle of step k follows every wave's wait for step k+1, which half B then reads.
// The prologue issues steps 0-2 and waits for step 0.  Loads of steps past the last have
// every offset out of range and write zeros into stages no later read uses.
//
// A wave issues at most one instruction per issue cycle of its SIMD, and an MFMA of this shape
// keeps the matrix unit busy for 8 of them, so the scalar and address work between two MFMAs
// stalls the unit once it exceeds 7 instructions.  The per-step work is therefore kept small
// (byte counts in 32 bits, see DmaCount), and the 8-wave form, which has registers to spare,
// runs the loop unrolled over the ring's four stages so that every LDS address of a step is a
// constant offset (kstep with S >= 0); in the 4-wave form that unrolling runs out of registers,
// so it computes the stage from k.
template <class W, bool A_CONTIG, bool B_CONTIG, bool RAGGED, int AG, int S>
__device__ __attribute__((always_inline)) inline void kstep(uint16_t *lds, const TileArgs &ta,
                                                            f32x16 (&acc)[W::TM][W::TN],
                                                            Frags<W> &F0, Frags<W> &F1,
                                                            GatherS &gs, int k, int wi, int wj,
                                                            int lane) {
  constexpr int TM = W::TM, TN = W::TN, NB = W::blk;
  const int nk = ta.nk;
  const int s0 = S >= 0 ? S : (k & 3);
  const uint16_t *cur = lds + s0 * STAGE_ELEMS;
  const uint16_t *nxt = lds + ((s0 + 1) & 3) * STAGE_ELEMS;
  const uint32_t st = (uint32_t)(uintptr_t)(lds_vptr)(lds + ((s0 + 3) & 3) * STAGE_ELEMS);
  __amdgpu_buffer_rsrc_t ra, rb;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < TM * TN; ++i) {  // half A
    const int tm = i / TN, tn = i % TN;
    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F0.b[tn], F0.a[tm], acc[tm][tn], 0,
                                                          0, 0);
    if (i < TM)
      F1.a[i] = read_operand<A_CONTIG>(cur, wi, i, lane, 1);
    else if (i < TM + TN)
      F1.b[i - TM] = read_operand<B_CONTIG>(cur + OP_ELEMS, wj, i - TM, lane, 1);
    // gathered strided operand: the other blocks' addresses of step k+3 (block 0's were
    // formed at the end of the previous step), ahead of their loads
    if constexpr (AG == 2) {
      static_assert(AG != 2 || NB == 2, "the gathered strided operand has two blocks per wave");
      if (i == 1) gather_s_addr_part<W>(gs, k + 3, 1, 0);
      if (i == 3) gather_s_addr_part<W>(gs, k + 3, 1, 1);
    }
    if (AG == 0 && i == 1) ra = dma_rsrc(ta.a, ta.ca, k + 3, nk);
    if (i == 2) rb = dma_rsrc(ta.b, ta.cb, k + 3, nk);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i == (u + 1) * TM * TN / (NB + 1)) {
        if constexpr (AG == 0)
          dma_one<W, A_CONTIG, RAGGED>(ta.a, ra, st, ta.wave_off, k + 3, ta.c_len, u);
        else if constexpr (AG == 1)
          gather_c_one<W>(ta.gc, st, ta.wave_off, k + 3, ta.c_len, u);
        else
          gather_s_one<W>(gs, st, ta.wave_off, u);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  waitcnt_vm<W::loads + NB>();
  __syncthreads();
  if constexpr (AG == 2) gather_s_fetch<W>(gs, k + 4);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < TM * TN; ++i) {  // half B
    const int tm = i / TN, tn = i % TN;
    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F1.b[tn], F1.a[tm], acc[tm][tn], 0,
                                                          0, 0);
    if (i < TM)
      F0.a[i] = read_operand<A_CONTIG>(nxt, wi, i, lane, 0);
    else if (i < TM + TN)
      F0.b[i - TM] = read_operand<B_CONTIG>(nxt + OP_ELEMS, wj, i - TM, lane, 0);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i == (u + 1) * TM * TN / (NB + 1))
        dma_one<W, B_CONTIG, RAGGED>(ta.b, rb, st + OP_ELEMS * 2, ta.wave_off, k + 3,
                                     ta.c_len, u);
    // gathered strided operand: addresses of step k+4 (issued in the next half A) from the
    // entries fetched after this step's barrier, once this half's fragment reads are out
    if constexpr (AG == 2) {
      if (i == TM * TN - 2) gather_s_addr_part<W>(gs, k + 4, 0, 0);
      if (i == TM * TN - 1) gather_s_addr_part<W>(gs, k + 4, 0, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <class W, bool A_CONTIG, bool B_CONTIG, bool RAGGED, int AG = 0>
__device__ inline void tile_mma(uint16_t *lds, TileArgs &ta, f32x16 (&acc)[W::TM][W::TN]) {
  constexpr int TM = W::TM, TN = W::TN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wi = (wid / W::N) * (32 * TM), wj = (wid % W::N) * (32 * TN);
  const int nk = ta.nk;
  if constexpr (AG == 0) ta.ca = dma_count(ta.a.bytes, ta.a.step);
  ta.cb = dma_count(ta.b.bytes, ta.b.step);
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (f32x16){};

  Frags<W> F0, F1;
  GatherS gs;
  if constexpr (AG == 2) gs = ta.gs;
#pragma unroll
  for (int kt = 0; kt < 3; ++kt) {
    if constexpr (AG == 2) {
      gather_s_fetch<W>(gs, kt);
      gather_s_addr<W>(gs, kt);
    }
    dma_step<W, A_CONTIG, B_CONTIG, RAGGED, AG>(lds, kt, ta, gs, kt);
  }
  if constexpr (AG == 2) {  // for the first half A, which issues step 3
    gather_s_fetch<W>(gs, 3);
    gather_s_addr<W>(gs, 3);
  }
  waitcnt_vm<2 * W::loads>();
  __syncthreads();
  read_frags<W, A_CONTIG, B_CONTIG>(F0, lds, wi, wj, lane, 0);
  if constexpr (W::n == 4) {
    for (int k = 0; k < nk; ++k)
      kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, -1>(lds, ta, acc, F0, F1, gs, k, wi, wj, lane);
  } else {
    int k = 0;
    for (; k + 4 <= nk; k += 4) {
      kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 0>(lds, ta, acc, F0, F1, gs, k, wi, wj, lane);
      kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 1>(lds, ta, acc, F0, F1, gs, k + 1, wi, wj, lane);
      kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 2>(lds, ta, acc, F0, F1, gs, k + 2, wi, wj, lane);
      kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 3>(lds, ta, acc, F0, F1, gs, k + 3, wi, wj, lane);
    }
    if (k < nk) {  // the last nk % 4 steps, from stage 0
      kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 0>(lds, ta, acc, F0, F1, gs, k, wi, wj, lane);
      if (k + 1 < nk) {
        kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 1>(lds, ta, acc, F0, F1, gs, k + 1, wi, wj,
                                                    lane);
        if (k + 2 < nk)
          kstep<W, A_CONTIG, B_CONTIG, RAGGED, AG, 2>(lds, ta, acc, F0, F1, gs, k + 2, wi, wj,
                                                      lane);
      }
    }
  }
  waitcnt_vm<0>();  // the trailing out-of-range loads land before the stages are reused
  __syncthreads();
}

// ---- DGRAD: 64-wide K stages ----------------------------------------------------------
// Both DGRAD operands are contiguous along the contraction, and at K steps of 32 each
// direct-to-LDS instruction of such an operand covers 16 rows x 64 B (16 half cache lines):
// the texture addresser, not the matrix units, then limits the loop (busy ~88% of the cycles
// against ~55% in FWD, whose weight operand comes in 512-byte rows).  DGRAD therefore loads
// 64-wide K stages, 8 rows x 128 B per instruction, in a ring of two 64-KB stages.  16-byte
// chunk k (0..7) of row r sits at position k ^ ((r >> 1) & 7), which keeps the fragment reads
// (16 rows per 256 B of banks) conflict-free.  (The FWD loop measured slower in this form:
// its weight operand already moves whole lines, and two stages give the loads less lead than
// the four-stage ring.)
constexpr int BK64 = 64;
constexpr int OP64_ELEMS = 256 * BK64;      // one operand of one stage
constexpr int STAGE64_ELEMS = 2 * OP64_ELEMS;
constexpr int kMaxBlk64 = 8;

struct DmaOp64 {
  const char *base;   // byte address of element (row 0, contraction 0) of the tile
  long long bytes;    // bytes readable from base
  int voff[kMaxBlk64];  // per-lane byte offset of this wave's blocks, or kOOB
  int kc[kMaxBlk64];    // contraction index of each block's chunk within a stage
};

template <class W>
__device__ inline void dma_init64(DmaOp64 &d, const uint16_t *base, long long bytes, int ld,
                                  int row_lim) {
  constexpr int NB = 32 / W::n;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  d.base = (const char *)base;
  d.bytes = bytes;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int blk = u * W::n + wid;        // 1-KB block of the 32-KB operand tile
    const int o = blk * 1024 + lane * 16;  // this lane's LDS byte offset
    const int r = o >> 7, p = (o >> 4) & 7;
    const int k = p ^ ((r >> 1) & 7);
    d.voff[u] = r < row_lim ? (r * ld + k * 8) * 2 : kOOB;
    d.kc[u] = k * 8;
  }
}

// Buffer resource of stage kt (a zero-byte resource past the last stage); c from
// dma_count(d.bytes, BK64 * 2).
__device__ inline __amdgpu_buffer_rsrc_t dma_rsrc64(const DmaOp64 &d, const DmaCount &c, int kt,
                                                    int nk) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(d.base + (long long)kt * BK64 * 2),
                                           (short)0, dma_bytes_at(c, BK64 * 2, kt, nk),
                                           0x00020000);
}

template <class W, bool RAGGED>
__device__ inline void dma_one64(const DmaOp64 &d, __amdgpu_buffer_rsrc_t rs, uint32_t lds_op,
                                 uint32_t wave_off, int kt, int c_lim, int u) {
  int off = d.voff[u];
  if (RAGGED) off = kt * BK64 + d.kc[u] < c_lim ? off : kOOB;
  // as dma_one: direct-to-LDS load at M0 + 16 * lane, one wait state after the M0 write
  const uint32_t m0 = lds_op + wave_off + u * W::n * 1024;
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off),
      "s"(rs), "{m0}"(m0)
      : "memory");
}

// MFMA operand t of lane `lane` at contraction 16 ks + 8 (lane / 32) .. +8 of the stage.
__device__ inline bf16x8 read_operand64(const uint16_t *src, int wbase, int t, int lane, int ks) {
  const int r = wbase + 32 * t + (lane & 31);
  const int k = 2 * ks + (lane >> 5);
  const int p = k ^ ((r >> 1) & 7);
  return __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + r * BK64 + p * 8));
}

struct TileArgs64 {
  DmaOp64 a, b;
  int c_len, nk;      // contraction length from the first stage, stages
  uint32_t wave_off;  // this wave's 1-KB block offset within an operand tile (wave-uniform)
};

// One 256x256 output tile from two contiguous operands, stage s in LDS stage s % 2.  Stage s:
// sub-steps 0..3 of 16, TM*TN MFMAs each; sub-steps 0-2 read the next sub-step's fragments
// and sub-step 0 issues the column-side loads of stage s+1 (its row-side loads went out in
// sub-step 3 of stage s-1); after sub-step 2 each wave waits for its loads (stage s+1) and a
// barrier follows, after which stage s+1 has landed everywhere and stage s has been read
// everywhere (the barrier waits for this wave's LDS reads); sub-step 3 reads stage s+1's first
// fragments and issues the row-side loads of stage s+2 into stage s's buffer.  The prologue
// issues stage 0 and the row side of stage 1 and waits for stage 0.  Loads of stages past the
// last write zeros into buffers no later read uses.  The buffer resources of stage s+2 are
// built in sub-steps 1 (row side) and 2 (column side, after stage s's last column-side load),
// whose MFMA slots have room for them (see tile_mma on issue slots).
template <class W, bool RAGGED>
__device__ inline void tile_mma64(uint16_t *lds, const TileArgs64 &ta,
                                  f32x16 (&acc)[W::TM][W::TN]) {
  constexpr int TM = W::TM, TN = W::TN, NB = 32 / W::n;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wi = (wid / W::N) * (32 * TM), wj = (wid % W::N) * (32 * TN);
  const int nk = ta.nk;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (f32x16){};
  auto stage_addr = [&](int s) {
    return (uint32_t)(uintptr_t)(lds_vptr)(lds + (s & 1) * STAGE64_ELEMS);
  };
  const DmaCount ca = dma_count(ta.a.bytes, BK64 * 2), cb = dma_count(ta.b.bytes, BK64 * 2);
  {
    const __amdgpu_buffer_rsrc_t ra0 = dma_rsrc64(ta.a, ca, 0, nk);
    const __amdgpu_buffer_rsrc_t rb0 = dma_rsrc64(ta.b, cb, 0, nk);
    const __amdgpu_buffer_rsrc_t ra1 = dma_rsrc64(ta.a, ca, 1, nk);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      dma_one64<W, RAGGED>(ta.a, ra0, stage_addr(0), ta.wave_off, 0, ta.c_len, u);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      dma_one64<W, RAGGED>(ta.b, rb0, stage_addr(0) + OP64_ELEMS * 2, ta.wave_off, 0, ta.c_len,
                           u);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      dma_one64<W, RAGGED>(ta.a, ra1, stage_addr(1), ta.wave_off, 1, ta.c_len, u);
  }
  waitcnt_vm<NB>();
  __syncthreads();
  Frags<W> F0, F1;
#pragma unroll
  for (int t = 0; t < TM; ++t) F0.a[t] = read_operand64(lds, wi, t, lane, 0);
#pragma unroll
  for (int t = 0; t < TN; ++t) F0.b[t] = read_operand64(lds + OP64_ELEMS, wj, t, lane, 0);
  __amdgpu_buffer_rsrc_t rb = dma_rsrc64(ta.b, cb, 1, nk);
  for (int s = 0; s < nk; ++s) {
    const uint16_t *cur = lds + (s & 1) * STAGE64_ELEMS;
    const uint16_t *nxt = lds + ((s + 1) & 1) * STAGE64_ELEMS;
    __amdgpu_buffer_rsrc_t ra;
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {  // sub-steps 0..2
      Frags<W> &Fc = (ks & 1) ? F1 : F0;
      Frags<W> &Fn = (ks & 1) ? F0 : F1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM * TN; ++i) {
        const int tm = i / TN, tn = i % TN;
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Fc.b[tn], Fc.a[tm], acc[tm][tn], 0,
                                                              0, 0);
        if (i < TM)
          Fn.a[i] = read_operand64(cur, wi, i, lane, ks + 1);
        else if (i < TM + TN)
          Fn.b[i - TM] = read_operand64(cur + OP64_ELEMS, wj, i - TM, lane, ks + 1);
        // the resources of the next loads, in slots with room (empty asms pin them there:
        // left alone, the compiler moves the arithmetic ahead of the stage's first MFMAs)
        if (ks == 1 && i == TM * TN - 4) {
          int kk = s + 2;
          asm volatile("" : "+s"(kk));
          ra = dma_rsrc64(ta.a, ca, kk, nk);
          asm volatile("" : "+s"(ra));
        }
        if (ks == 2 && i == TM * TN - 4) {  // after this stage's last column-side load
          int kk = s + 2;
          asm volatile("" : "+s"(kk));
          rb = dma_rsrc64(ta.b, cb, kk, nk);
          asm volatile("" : "+s"(rb));
        }
        if (ks == 0) {
#pragma unroll
          for (int u = 0; u < NB; ++u)
            if (i == (u + 1) * TM * TN / (NB + 1))
              dma_one64<W, RAGGED>(ta.b, rb, stage_addr(s + 1) + OP64_ELEMS * 2, ta.wave_off,
                                   s + 1, ta.c_len, u);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    waitcnt_vm<0>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {  // sub-step 3
      const int tm = i / TN, tn = i % TN;
      acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F1.b[tn], F1.a[tm], acc[tm][tn], 0,
                                                            0, 0);
      if (i < TM)
        F0.a[i] = read_operand64(nxt, wi, i, lane, 0);
      else if (i < TM + TN)
        F0.b[i - TM] = read_operand64(nxt + OP64_ELEMS, wj, i - TM, lane, 0);
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (i == (u + 1) * TM * TN / (NB + 1))
          dma_one64<W, RAGGED>(ta.a, ra, stage_addr(s + 2), ta.wave_off, s + 2, ta.c_len, u);

      __builtin_amdgcn_sched_barrier(0);
    }
  }
  waitcnt_vm<0>();  // the trailing out-of-range loads land before the stages are reused
  __syncthreads();
}

// Decode a tile index into (row tile, col tile) walking groups of kGroupM row tiles.
__device__ inline void swizzle(int t, int n_rt, int n_ct, int *rt, int *ct) {
  const int per_group = kGroupM * n_ct;
  const int g = t / per_group;
  const int r = t - g * per_group;
  const int gm = min(kGroupM, n_rt - g * kGroupM);
  *rt = g * kGroupM + r % gm;
  *ct = r / gm;
}

__device__ inline int logical_block() {
  // workgroups are dealt round-robin to the XCDs; give each XCD a contiguous range
  const int b = blockIdx.x, n = gridDim.x;
  if (n % kXcds) return b;
  return (b % kXcds) * (n / kXcds) + b / kXcds;
}

// Segment table: sCu[rho] (clamped to [0, M_total]) and sStart[rho] = first row tile of rho.
template <class W>
__device__ inline int build_tiles(const int32_t *cu, int G, int M_total, int *sCu, int *sStart,
                                  bool wgrad) {
  __shared__ int tmp[W::n];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i <= G; i += W::threads) sCu[i] = min(max(cu[i], 0), M_total);
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < G; base += W::threads) {
    const int rho = base + tid;
    int v = 0;
    if (rho < G) {
      const int n = sCu[rho + 1] - sCu[rho];
      v = n > 0 ? (wgrad ? 1 : (n + BM - 1) / BM) : 0;
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < W::n; ++w) {
      before += w < wid ? tmp[w] : 0;
      tot += tmp[w];
    }
    const int carry = carry_s;
    if (rho < G) sStart[rho] = carry + before + x - v;
    __syncthreads();
    if (tid == 0) carry_s = carry + tot;
    __syncthreads();
  }
  const int total = carry_s;
  if (tid == 0) sStart[G] = total;
  __syncthreads();
  return total;
}

// last rho with sStart[rho] <= t (the segment owning row tile t)
__device__ inline int find_seg(const int *sStart, int G, int t) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sStart[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// sOrd[i] = index (among the non-empty segments, as sStart counts them for WGRAD) of the
// i-th longest non-empty segment; ties keep segment order.  tmp: n_ne ints of scratch LDS.
template <class W>
__device__ inline void order_by_length(const int *sCu, const int *sStart, int G, int n_ne,
                                       int *sOrd, int *tmp) {
  const int tid = threadIdx.x;
  for (int rho = tid; rho < G; rho += W::threads) {
    const int len = sCu[rho + 1] - sCu[rho];
    if (len > 0) tmp[sStart[rho]] = len;
  }
  __syncthreads();
  for (int i = tid; i < n_ne; i += W::threads) {
    const int len = tmp[i];
    int rank = 0;
    for (int j = 0; j < n_ne; ++j) {
      const int l = tmp[j];
      rank += l > len || (l == len && j < i);
    }
    sOrd[rank] = i;
  }
  __syncthreads();
}

// bf16 output-tile epilogue.  The accumulator layout leaves each lane 4 consecutive columns
// of one row, so a store straight from registers writes 32 rows x 16 B per instruction.
// The tile goes through LDS instead (free once the K loop has drained): each wave writes its
// fragments, then the whole 256 x 256 tile (128 KB) leaves in row segments of 16 B per lane,
// 512 B of one row per 32 lanes.  16-byte LDS chunks are XOR-swizzled by row so the
// fragment writes spread over the banks and the row reads are conflict-free.  Rows >= rows
// and columns >= cols of the tile are not written (cols is a multiple of 8).
template <class W>
__device__ inline void epilogue_bf16(uint16_t *lds, const f32x16 (&acc)[W::TM][W::TN],
                                     uint16_t *o, long long ld, int rows, int cols, int wi,
                                     int wj, int lane, int wid) {
#pragma unroll
  for (int tm = 0; tm < W::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < W::TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = wi + tm * 32 + (lane & 31);
        const int c = (wj + tn * 32 + g * 8) >> 3;  // 8-column chunk
        const f32x16 &a = acc[tm][tn];
        uint2 v;
        v.x = pack_bf16x2(a[4 * g + 0], a[4 * g + 1]);
        v.y = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
        *(uint2 *)(lds + i * 256 + (c ^ (i & 31)) * 8 + (lane >> 5) * 4) = v;
      }
  __syncthreads();
  constexpr int kRows = BM / W::n;  // rows stored by one wave, two per instruction
  // the row offsets below depend only on the lane; left alone, the compiler computes them
  // once per kernel and spills them across the K loop (the empty asm makes it recompute them
  // per tile, a few instructions)
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int r = 0; r < kRows / 2; ++r) {
    const int i = wid * kRows + 2 * r + (ln >> 5);
    const int c = ln & 31;
    const u32x4 v = *(const u32x4 *)(lds + i * 256 + (c ^ (i & 31)) * 8);
    if (i < rows && c * 8 < cols) *(u32x4 *)(o + i * ld + c * 8) = v;
  }
  __syncthreads();
}

// Gated (SwiGLU) output: W's columns come in (gate, up) pairs, so each lane's 4 consecutive
// accumulator columns hold two pairs and z = silu(gate) * up is register-local.  The 256 x 128
// z tile (64 KB bf16) leaves through LDS like the bf16 epilogue: chunk (8 z values) c of row i
// at c ^ (i & 15), then 16-byte row segments, 256 B per row.  cols (valid z columns of the
// tile) is a multiple of 8.
constexpr int kOpSwiglu = 3;  // internal op: FWD main loop, gated epilogue

__device__ inline float silu_f32(float x) { return x / (1.0f + __expf(-x)); }

template <class W>
__device__ inline void epilogue_swiglu(uint16_t *lds, const f32x16 (&acc)[W::TM][W::TN],
                                       uint16_t *o, long long ld, int rows, int cols, int wi,
                                       int wj, int lane) {
#pragma unroll
  for (int tm = 0; tm < W::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < W::TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = wi + tm * 32 + (lane & 31);
        const int jz = (wj + tn * 32 + g * 8 + (lane >> 5) * 4) >> 1;  // even z column
        const f32x16 &a = acc[tm][tn];
        const uint32_t v = pack_bf16x2(silu_f32(a[4 * g + 0]) * a[4 * g + 1],
                                       silu_f32(a[4 * g + 2]) * a[4 * g + 3]);
        *(uint32_t *)(lds + i * 128 + ((jz >> 3) ^ (i & 15)) * 8 + (jz & 7)) = v;
      }
  __syncthreads();
  constexpr int kPass = W::threads / 16;  // rows per pass, 16 chunks each
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // per-tile row offsets, as in epilogue_bf16
#pragma unroll
  for (int r = 0; r < BM / kPass; ++r) {
    const int i = (tid >> 4) + kPass * r;
    const int c = tid & 15;
    const u32x4 v = *(const u32x4 *)(lds + i * 128 + (c ^ (i & 15)) * 8);
    if (i < rows && c * 8 < cols) *(u32x4 *)(o + i * ld + c * 8) = v;
  }
  __syncthreads();
}

// WGRAD epilogue: fp32 out += acc for the `rows` x `cols` part of the tile inside the output,
// staged through LDS (free once the K loop has drained) so that global memory sees whole rows.
// Two passes; in pass p every wave writes its row blocks tm = 2p, 2p+1 into LDS (tile rows
// 64p .. 64p+63 and 128+64p .. 128+64p+63: 128 rows x 1 KB) and issues its loads of the old
// values, then after a barrier every thread adds and stores its 16-byte chunks, a wave
// instruction covering one whole 1-KB row.  A chunk outside the output (a row at or past
// `rows`, or columns at or past `cols`) takes a per-lane offset past the buffer resource, so
// its load returns zero and its store is dropped: a tile cut by the edge needs no separate
// code path (the per-element register form it replaced also cost the kernel ~30 registers
// and 1-2%).  Compared with read-modify-writes straight from the accumulator layout (32 bytes
// of each of 32 rows per instruction) this sends 8x fewer requests to L2 for the same bytes;
// the old values are read and written non-temporally (each is touched once per call).  LDS
// rows are padded to kRmwLd floats, which spreads the 32 rows a wave writes per instruction
// over all banks.
constexpr int kRmwLd = 260;
constexpr int kRmwLdsElems = 2 * 128 * kRmwLd;  // bf16 elements of the staging area
constexpr int kNonTemporal = 2;                 // cache-policy bit of buffer loads and stores

template <class W>
__device__ inline void wgrad_rmw(float *o, int N, int rows, int cols,
                                 const f32x16 (&acc)[W::TM][W::TN], uint16_t *lds_raw, int wi,
                                 int wj, int lane) {
  constexpr int TN = W::TN;
  static_assert(W::TM == 4, "128-row wave blocks");
  constexpr int RS = W::threads / 64;   // staged rows per pass of all threads (one per wave)
  constexpr int Q = 128 / RS;           // staged rows per thread and pass
  float *L = (float *)lds_raw;  // 128 rows x kRmwLd floats
  const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;  // chunk, first staged row (+RS q)
  // One resource over the tile's rows; the row of each load and store goes in the
  // (wave-uniform) scalar offset, the chunk's column in the per-lane offset.  Chunks outside
  // the output get the per-lane offset kOOB, which is past the resource whether or not the
  // hardware's range check counts the scalar offset (kOOB + any row offset of a tile stays
  // below 2^32: rows < 256 and N <= 2^20).
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(o, ((long long)rows * N - (N - cols)) * 4);
  const int voff = c * 4 < cols ? (r0 * N + c * 4) * 4 : kOOB;
  float *wr = L + ((wi >> 1) + (lane & 31)) * kRmwLd + wj + (lane >> 5) * 4;
  const float *rd = L + r0 * kRmwLd + c * 4;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16 &a = acc[2 * p + b][tn];
          const f32x4 v = {a[4 * g + 0], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          *(f32x4 *)(wr + b * 32 * kRmwLd + tn * 32 + g * 8) = v;
        }
    // staged row r0 + RS q (q < Q) holds tile row r0 + trow(q): the first Q/2 staged rows are
    // tile rows 64p .., the last Q/2 are tile rows 128 + 64p ..
    constexpr int QB = Q < 16 ? Q : 16;  // old values held per batch
    u32x4 old[QB];
    auto trow = [&](int q) { return (q < Q / 2 ? 64 * p : 64 + 64 * p) + RS * q; };
    auto soff = [&](int q) { return trow(q) * N * 4; };
    auto vof = [&](int q) { return r0 + trow(q) < rows ? voff : kOOB; };
#pragma unroll
    for (int q = 0; q < QB; ++q)
      old[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vof(q), soff(q), kNonTemporal);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < Q / QB; ++b) {
      if (b > 0) {
#pragma unroll
        for (int q = 0; q < QB; ++q)
          old[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vof(b * QB + q), soff(b * QB + q),
                                                         kNonTemporal);
      }
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const f32x4 a = *(const f32x4 *)(rd + RS * (b * QB + q) * kRmwLd);
        f32x4 v = __builtin_bit_cast(f32x4, old[q]);
        v[0] += a[0];
        v[1] += a[1];
        v[2] += a[2];
        v[3] += a[3];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                               vof(b * QB + q), soff(b * QB + q), kNonTemporal);
      }
    }
    __syncthreads();
  }
}

// Per-workgroup constants of the tile loops.
struct TileCtx {
  int lane, wid, wi, wj;
  uint32_t wave_off;  // this wave's 1-KB block offset within an operand tile (wave-uniform)
};

template <class W>
__device__ inline TileCtx tile_ctx() {
  TileCtx c;
  c.lane = threadIdx.x & 63;
  c.wid = threadIdx.x >> 6;
  c.wi = (c.wid / W::N) * (32 * W::TM);
  c.wj = (c.wid % W::N) * (32 * W::TN);
  c.wave_off = __builtin_amdgcn_readfirstlane(c.wid) * 1024;
  return c;
}

// Split of the last, partial round of row-operand tiles (data-parallel rounds + a split
// round).  The T output tiles of a row-operand GEMM all take nk K steps; the persistent grid
// deals them round-robin, so when T is not a multiple of the grid the last round keeps only
// L = T mod grid workgroups busy for a whole tile.  With a workspace the first F = T - L
// tiles are dealt as before and each leftover tile u is cut into P equal K ranges (P =
// grid / L, at least kSkMinPart of contraction each): workgroup c = p L + u (in the XCD-grouped
// order of logical_block) takes part p of tile u and stores its fp32 accumulators into
// workspace slot c; a second kernel adds each tile's P parts in K order and runs the tile's
// usual epilogue.  Part-major numbering puts the same K range of neighbouring tiles on one
// XCD, so the split round shares operand panels in L2 as a whole round does.  The split is
// taken only when it saves more than kSkGain of contraction in the last round.
constexpr int kSkGain = 1536;     // contraction the split must save (covers its store and reduce)
constexpr int kSkMinPart = 512;   // contraction per part at least
constexpr int kTileFloats = BM * BN;

// Width of a K stage of the row-operand GEMMs: 64 for DGRAD (see tile_mma64), else 32.
template <int OP>
constexpr int kStageK = OP == MOE_GEMM_DGRAD ? BK64 : BK;

struct SkPlan {
  int F, L, P, nk;  // whole tiles, leftover tiles, parts per leftover tile, K stages per tile
  bool on;
  __device__ int k_begin(int p) const { return (int)((long long)p * nk / P); }
};

// nk K stages of width bk per tile
__device__ inline SkPlan sk_plan(long long T, int nk, int bk, int grid, bool allowed) {
  SkPlan s;
  s.F = (int)T;
  s.L = 0;
  s.P = 1;
  s.nk = nk;
  s.on = false;
  const int L = (int)(T % grid);
  if (!allowed || L == 0 || (long long)nk * bk * (grid - L) <= (long long)kSkGain * grid)
    return s;
  const int P = min(grid / L, nk * bk / kSkMinPart);
  if (P < 2) return s;
  s.on = true;
  s.F = (int)(T - L);
  s.L = L;
  s.P = P;
  return s;
}

// Partial accumulators of one tile in a workspace slot: 16-byte chunk i = (tm TN + tn) 4 + g
// of thread x at slot + (i threads + x) 4 floats, so each wave instruction moves 1 KB.
template <class W>
__device__ inline void store_partial(float *__restrict__ slot, const f32x16 (&acc)[W::TM][W::TN]) {
#pragma unroll
  for (int tm = 0; tm < W::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < W::TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = (tm * W::TN + tn) * 4 + g;
        const f32x4 v = {acc[tm][tn][4 * g], acc[tm][tn][4 * g + 1], acc[tm][tn][4 * g + 2],
                         acc[tm][tn][4 * g + 3]};
        *(f32x4 *)(slot + ((size_t)i * W::threads + threadIdx.x) * 4) = v;
      }
}

template <class W>
__device__ inline void add_partial(f32x16 (&acc)[W::TM][W::TN], const float *__restrict__ slot) {
#pragma unroll
  for (int tm = 0; tm < W::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < W::TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = (tm * W::TN + tn) * 4 + g;
        const f32x4 v = *(const f32x4 *)(slot + ((size_t)i * W::threads + threadIdx.x) * 4);
        acc[tm][tn][4 * g] += v[0];
        acc[tm][tn][4 * g + 1] += v[1];
        acc[tm][tn][4 * g + 2] += v[2];
        acc[tm][tn][4 * g + 3] += v[3];
      }
}

// Where output tile t of a row-operand GEMM lies: segment rho, first row m0, rows, first
// output column j0 (row tiles of each segment from sStart, column tiles from n_ct).
struct RowsTile {
  int rho, m0, rows, j0;
};

__device__ inline RowsTile rows_tile_at(int t, int G, int n_rt_total, int n_ct, const int *sCu,
                                        const int *sStart) {
  RowsTile r;
  int rt, ct;
  swizzle(t, n_rt_total, n_ct, &rt, &ct);
  r.rho = find_seg(sStart, G, rt);
  r.m0 = sCu[r.rho] + (rt - sStart[r.rho]) * BM;
  r.rows = min(BM, sCu[r.rho + 1] - r.m0);
  r.j0 = ct * BN;
  return r;
}

// The output-tile epilogue of the row-operand GEMMs.
template <int OP, class W>
__device__ inline void rows_epilogue(uint16_t *lds, const f32x16 (&acc)[W::TM][W::TN],
                                     void *__restrict__ out, void *__restrict__ out2, int Kd,
                                     int N, const RowsTile &r, const TileCtx &cx) {
  if (OP == kOpSwiglu) {
    // out = z [M, N/2], out2 = pre-activation h [M, N] (optional)
    if (out2)
      epilogue_bf16<W>(lds, acc, (uint16_t *)out2 + (size_t)r.m0 * N + r.j0, N, r.rows,
                       N - r.j0, cx.wi, cx.wj, cx.lane, cx.wid);
    epilogue_swiglu<W>(lds, acc, (uint16_t *)out + (size_t)r.m0 * (N / 2) + r.j0 / 2, N / 2,
                       r.rows, (N - r.j0) / 2, cx.wi, cx.wj, cx.lane);
  } else {
    const int ncols = OP == MOE_GEMM_DGRAD ? Kd : N;
    epilogue_bf16<W>(lds, acc, (uint16_t *)out + (size_t)r.m0 * ncols + r.j0, ncols, r.rows,
                     ncols - r.j0, cx.wi, cx.wj, cx.lane, cx.wid);
  }
}

// K steps [k0, k1) of output tile t of the row-operand GEMMs (FWD, DGRAD, gated FWD): rows of
// one segment x 256 output columns.  FWD: out[m, j] = sum_c a[m, c] W[rho][c, j], c < Kd.
// DGRAD: out[m, j] = sum_c a[m, c] W[rho][j, c], c < N, j < Kd.  The whole contraction ends
// in the epilogue; a part of it is stored to `partial` instead.
// With GATHER (FWD and the gated FWD only), the rows come from the token rows through gp.
template <int OP, bool RAGGED, class W, bool GATHER>
__device__ inline void rows_tile(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                                 void *__restrict__ out, void *__restrict__ out2, int G, int Kd,
                                 int N, int n_rt_total, int n_ct, const int *sCu,
                                 const int *sStart, uint16_t *lds, int t, int k0, int k1,
                                 float *__restrict__ partial, const TileCtx &cx,
                                 const GatherParams &gp) {
  f32x16 acc[W::TM][W::TN];
  const RowsTile r = rows_tile_at(t, G, n_rt_total, n_ct, sCu, sStart);
  const uint16_t *w = b + (size_t)r.rho * Kd * N;
  // K stages [k0, k1): both operands start k0 stages in (loads of stages past k1 - k0 read
  // nothing), and the contraction length left for the ragged last stage shrinks to match
  if constexpr (OP == MOE_GEMM_DGRAD) {
    TileArgs64 ta;
    ta.wave_off = cx.wave_off;
    dma_init64<W>(ta.a, a + (size_t)r.m0 * N, (long long)r.rows * N * 2, N, r.rows);
    dma_init64<W>(ta.b, w + (size_t)r.j0 * N, (long long)(Kd - r.j0) * N * 2, N, Kd - r.j0);
    const long long d0 = (long long)k0 * BK64 * 2;
    ta.a.base += d0;
    ta.a.bytes -= d0;
    ta.b.base += d0;
    ta.b.bytes -= d0;
    ta.c_len = N - k0 * BK64;
    ta.nk = k1 - k0;
    tile_mma64<W, RAGGED>(lds, ta, acc);
  } else {
    TileArgs ta;
    ta.wave_off = cx.wave_off;
    if constexpr (GATHER) {
      gather_c_init<W>(ta.gc, gp, r.m0, r.rows, k0);
    } else {
      dma_init<W, true>(ta.a, a + (size_t)r.m0 * Kd, (long long)r.rows * Kd * 2, Kd, r.rows);
      const long long da = (long long)k0 * ta.a.step;
      ta.a.base += da;
      ta.a.bytes -= da;
    }
    dma_init<W, false>(ta.b, w + r.j0, ((long long)Kd * N - r.j0) * 2, N, N - r.j0);
    const long long db = (long long)k0 * ta.b.step;
    ta.b.base += db;
    ta.b.bytes -= db;
    ta.c_len = Kd - k0 * BK;
    ta.nk = k1 - k0;
    tile_mma<W, true, false, RAGGED, GATHER ? 1 : 0>(lds, ta, acc);
  }
  if (partial)
    store_partial<W>(partial, acc);
  else
    rows_epilogue<OP, W>(lds, acc, out, out2, Kd, N, r, cx);
}

// Output tile t of the weight-gradient GEMM: out[rho][i, j] += sum_m a[m, i] b[m, j] over
// the rows m of segment rho, i < Kd, j < N; n_it x n_ct tiles per active segment (sStart:
// index of each segment among the active ones).
// With GATHER, row m of the first operand is a token row of gp.
template <class W, bool GATHER>
__device__ inline void wgrad_tile(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                                  float *__restrict__ out, int G, int Kd, int N, int n_it,
                                  int n_ct, const int *sCu, const int *sStart, const int *sOrd,
                                  uint16_t *lds, long long t, const TileCtx &cx,
                                  const GatherParams &gp) {
  constexpr int TM = W::TM, TN = W::TN;
  f32x16 acc[TM][TN];
  const int per_seg = n_it * n_ct;
  const int sidx = (int)(t / per_seg);
  int it, ct;
  swizzle((int)(t - (long long)sidx * per_seg), n_it, n_ct, &it, &ct);
  const int rho = find_seg(sStart, G, sOrd[sidx]);
  const int m0 = sCu[rho], len = sCu[rho + 1] - m0;
  const int i0 = it * BM, j0 = ct * BN;
  TileArgs ta;
  ta.wave_off = cx.wave_off;
  if constexpr (GATHER)
    gather_s_init<W>(ta.gs, gp, m0, len, i0, Kd);
  else
    dma_init<W, false>(ta.a, a + (size_t)m0 * Kd + i0, ((long long)len * Kd - i0) * 2, Kd,
                       Kd - i0);
  dma_init<W, false>(ta.b, b + (size_t)m0 * N + j0, ((long long)len * N - j0) * 2, N, N - j0);
  ta.c_len = len;
  ta.nk = (len + BK - 1) / BK;
  tile_mma<W, false, false, false, GATHER ? 2 : 0>(lds, ta, acc);
  float *o = out + ((size_t)rho * Kd + i0) * N + j0;
  wgrad_rmw<W>(o, N, Kd - i0, N - j0, acc, lds, cx.wi, cx.wj, cx.lane);
}

// LDS of the tile loops: the K loop's ring; the WGRAD epilogue stages through a slightly
// larger area.
constexpr int kLdsRing = kStages * STAGE_ELEMS;
constexpr int kLdsWgrad = kRmwLdsElems > kLdsRing ? kRmwLdsElems : kLdsRing;

// GATHER: the row operand (FWD, gated FWD) or the first operand (WGRAD) is read from token
// rows through gp instead of from `a`.
template <int OP, bool RAGGED, int WN, bool GATHER = false>
__global__ __launch_bounds__(Waves<WN>::threads, 1) void k_ggemm_bf16(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
    const int32_t *__restrict__ cu, void *__restrict__ out, void *__restrict__ out2,
    float *__restrict__ ws, int G, int M_total, int Kd, int N, GatherParams gp) {
  using W = Waves<WN>;
  constexpr bool wgrad = OP == MOE_GEMM_WGRAD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[wgrad ? kLdsWgrad : kLdsRing];
  __shared__ int sCu[kMaxG + 1], sStart[kMaxG + 1];
  const int n_rt_total = build_tiles<W>(cu, G, M_total, sCu, sStart, wgrad);
  // FWD: i = rows, j = n in [0,N), c = kd.  DGRAD: i = rows, j = kd, c = n.
  // WGRAD: i = kd, j = n, c = rows of the segment (per active segment: n_it x n_jt tiles).
  const int ncols = OP == MOE_GEMM_DGRAD ? Kd : N;
  const int n_ct = (ncols + BN - 1) / BN;
  const int n_it = (Kd + BM - 1) / BM;
  const long long total = wgrad ? (long long)n_rt_total * n_it * n_ct : (long long)n_rt_total * n_ct;
  const TileCtx cx = tile_ctx<W>();
  if constexpr (wgrad) {
    // A WGRAD tile's cost grows with its segment's row count.  Deal the segments longest
    // first and the rounds of tiles back and forth (snake), so the workgroups that drew long
    // tiles in one round draw short ones in the next; each XCD still takes 32 neighbouring
    // tiles per round.
    __shared__ int sOrd[kMaxG];
    order_by_length<W>(sCu, sStart, G, n_rt_total, sOrd, (int *)lds);
    const int lb = logical_block(), grid = gridDim.x;
    long long base = 0;
    for (int r = 0; base < total; ++r, base += grid) {
      const long long t = base + ((r & 1) ? grid - 1 - lb : lb);
      if (t < total)
        wgrad_tile<W, GATHER>(a, b, (float *)out, G, Kd, N, n_it, n_ct, sCu, sStart, sOrd, lds,
                              t, cx, gp);
    }
  } else {
    constexpr int bk = kStageK<OP>;
    const int nk = ((OP == MOE_GEMM_DGRAD ? N : Kd) + bk - 1) / bk;
    const SkPlan sk = sk_plan(total, nk, bk, gridDim.x, ws != nullptr);
    const int lb = logical_block();
    // whole tiles lb, lb + grid, .. < F, then (workgroups lb < L P) part lb / L of leftover
    // tile lb % L (one call site keeps one inlined copy of the tile code)
    int t = lb;
    bool part = sk.on && lb < sk.L * sk.P;
    for (;;) {
      int tile, k0 = 0, k1 = nk;
      float *slot = nullptr;
      if (t < sk.F) {
        tile = t;
        t += gridDim.x;
      } else if (part) {
        const int u = lb % sk.L, pp = lb / sk.L;
        tile = sk.F + u;
        k0 = sk.k_begin(pp);
        k1 = sk.k_begin(pp + 1);
        slot = ws + (size_t)lb * kTileFloats;
        part = false;
      } else {
        break;
      }
      rows_tile<OP, RAGGED, W, GATHER>(a, b, out, out2, G, Kd, N, n_rt_total, n_ct, sCu, sStart,
                                       lds, tile, k0, k1, slot, cx, gp);
    }
  }
}

// Second kernel of a split last round: adds the P parts of each leftover tile in K order
// (fp32) and writes the tile's outputs as its epilogue would, chunk by chunk.  A chunk is one
// 16-byte piece of a slot (4 consecutive output columns of one row, see store_partial), so
// the reads of the parts are contiguous across threads and every workgroup of the grid takes
// a share of every split tile.  Same tile table and, through gemm_grid, the same split as the
// GEMM (WN: its wave layout).  kSkReduceBlocks blocks per GEMM workgroup keep enough loads in
// flight.
constexpr int kSkReduceBlocks = 8;

template <int OP, int WN>
__global__ __launch_bounds__(256) void k_ggemm_sk_reduce(
    const int32_t *__restrict__ cu, void *__restrict__ out, void *__restrict__ out2,
    const float *__restrict__ ws, int gemm_grid, int G, int M_total, int Kd, int N) {
  using W = Waves<WN>;      // the GEMM's layout of the slots
  using B = Waves<2>;       // this kernel's 256 threads
  __shared__ int sCu[kMaxG + 1], sStart[kMaxG + 1];
  const int n_rt_total = build_tiles<B>(cu, G, M_total, sCu, sStart, false);
  const int ncols = OP == MOE_GEMM_DGRAD ? Kd : N;
  const int n_ct = (ncols + BN - 1) / BN;
  constexpr int bk = kStageK<OP>;
  const int nk = ((OP == MOE_GEMM_DGRAD ? N : Kd) + bk - 1) / bk;
  const SkPlan sk = sk_plan((long long)n_rt_total * n_ct, nk, bk, gemm_grid, true);
  if (!sk.on) return;
  constexpr int kChunks = kTileFloats / 4;
  const long long total = (long long)sk.L * kChunks;
  for (long long ch = (long long)blockIdx.x * B::threads + threadIdx.x; ch < total;
       ch += (long long)gridDim.x * B::threads) {
    const int u = (int)(ch / kChunks), e = (int)(ch - (long long)u * kChunks);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int pp = 0; pp < sk.P; ++pp)
      v += *(const f32x4 *)(ws + ((size_t)(pp * sk.L + u) * kTileFloats + (size_t)e * 4));
    // chunk e = i * threads + x of the GEMM's thread x: accumulator block (tm, tn), group g
    const int x = e % W::threads, i = e / W::threads;
    const int tm = i / (W::TN * 4), tn = (i / 4) % W::TN, g = i % 4;
    const int wid = x >> 6, lane = x & 63;
    const int row = (wid / W::N) * (32 * W::TM) + tm * 32 + (lane & 31);
    const int col = (wid % W::N) * (32 * W::TN) + tn * 32 + g * 8 + (lane >> 5) * 4;
    const RowsTile r = rows_tile_at(sk.F + u, G, n_rt_total, n_ct, sCu, sStart);
    if (row >= r.rows || r.j0 + col >= ncols) continue;
    const size_t m = (size_t)(r.m0 + row);
    if (OP == kOpSwiglu) {
      if (out2) {
        uint2 hv;
        hv.x = pack_bf16x2(v[0], v[1]);
        hv.y = pack_bf16x2(v[2], v[3]);
        *(uint2 *)((uint16_t *)out2 + m * N + r.j0 + col) = hv;
      }
      *(uint32_t *)((uint16_t *)out + m * (N / 2) + (r.j0 + col) / 2) =
          pack_bf16x2(silu_f32(v[0]) * v[1], silu_f32(v[2]) * v[3]);
    } else {
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *(uint2 *)((uint16_t *)out + m * ncols + r.j0 + col) = o;
    }
  }
}

// ---------------------------------------------------------------------------------------
// fp32 vector-ALU path (small shapes)
// ---------------------------------------------------------------------------------------

__device__ inline int seg_of_row(const int32_t *cu, int G, int row) {
  int lo = 0, hi = G;  // last rho with cu[rho] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <int OP>
__global__ __launch_bounds__(256) void k_ggemm_f32_rows(const float *__restrict__ a,
                                                        const float *__restrict__ w,
                                                        const int32_t *__restrict__ cu,
                                                        float *__restrict__ out, int G,
                                                        int M_total, int Kd, int N) {
  const int ncols = OP == MOE_GEMM_FWD ? N : Kd;
  const int kc = OP == MOE_GEMM_FWD ? Kd : N;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / ncols), col = (int)(idx % ncols);
  const int end = min(max(cu[G], 0), M_total);
  if (row >= end || row < max(cu[0], 0)) return;
  const int rho = seg_of_row(cu, G, row);
  if (row >= cu[rho + 1]) return;
  const float *wr = w + (size_t)rho * Kd * N;
  const float *ar = a + (size_t)row * kc;
  float s = 0.f;
  for (int c = 0; c < kc; ++c) {
    const float wv = OP == MOE_GEMM_FWD ? wr[(size_t)c * N + col] : wr[(size_t)col * N + c];
    s = __builtin_fmaf(ar[c], wv, s);
  }
  out[(size_t)row * ncols + col] = s;
}

__global__ __launch_bounds__(256) void k_ggemm_f32_wgrad(const float *__restrict__ a,
                                                         const float *__restrict__ bm,
                                                         const int32_t *__restrict__ cu,
                                                         float *__restrict__ out, int G,
                                                         int M_total, int Kd, int N) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per = (long long)Kd * N;
  if (idx >= per * G) return;
  const int rho = (int)(idx / per);
  const int i = (int)((idx % per) / N), j = (int)(idx % N);
  const int lo = min(max(cu[rho], 0), M_total), hi = min(max(cu[rho + 1], 0), M_total);
  if (hi <= lo) return;
  float s = 0.f;
  for (int m = lo; m < hi; ++m) s = __builtin_fmaf(a[(size_t)m * Kd + i], bm[(size_t)m * N + j], s);
  out[idx] += s;
}

}  // namespace moe

using namespace moe;

// Workspace of the split last round: one fp32 tile slot per workgroup of the persistent grid.
static size_t sk_workspace_bytes() { return (size_t)device_cu_count() * kTileFloats * 4; }

// A row-operand bf16 GEMM: the persistent kernel, then (when a workspace is given and the
// tiles are long enough that a split could pay) the reduce of the split last round.  The
// kernel decides on the device whether to split; the reduce returns at once when it did not.
// With GATHER the row operand is read through gp (a gathered load tests every chunk against
// the contraction's end itself, so it needs no RAGGED form).
template <int OP, int WN, bool GATHER = false>
static void launch_rows(int contraction, const uint16_t *a, const uint16_t *b,
                        const int32_t *cu, void *out, void *out2, void *ws, int G, int M_total,
                        int Kd, int N, hipStream_t stream, const GatherParams &gp = {}) {
  const int grid = device_cu_count();
  // a split can pay only when a tile's contraction exceeds what it must save
  float *sk_ws = ws && contraction > kSkGain ? (float *)ws : nullptr;
  // a contiguous operand whose contraction is not a multiple of the K stage needs a per-lane
  // column test in its last stage
  if constexpr (GATHER)
    hipLaunchKernelGGL((k_ggemm_bf16<OP, false, WN, true>), dim3(grid),
                       dim3(Waves<WN>::threads), 0, stream, a, b, cu, out, out2, sk_ws, G,
                       M_total, Kd, N, gp);
  else if (contraction % kStageK<OP> != 0)
    hipLaunchKernelGGL((k_ggemm_bf16<OP, true, WN>), dim3(grid), dim3(Waves<WN>::threads), 0,
                       stream, a, b, cu, out, out2, sk_ws, G, M_total, Kd, N, gp);
  else
    hipLaunchKernelGGL((k_ggemm_bf16<OP, false, WN>), dim3(grid), dim3(Waves<WN>::threads), 0,
                       stream, a, b, cu, out, out2, sk_ws, G, M_total, Kd, N, gp);
  if (sk_ws)
    hipLaunchKernelGGL((k_ggemm_sk_reduce<OP, WN>), dim3(grid * kSkReduceBlocks), dim3(256), 0,
                       stream, cu, out, out2, sk_ws, grid, G, M_total, Kd, N);
}

extern "C" size_t moe_group_gemm_workspace_bytes(moe_gemm_op op, moe_dtype dtype) {
  return dtype == MOE_BF16 && op != MOE_GEMM_WGRAD ? sk_workspace_bytes() : 0;
}

extern "C" moe_status_t moe_group_gemm(moe_gemm_op op, moe_dtype dtype, int32_t G,
                                       int32_t M_total, int32_t Kd, int32_t N, const void *a,
                                       const void *b, const int32_t *cu_seqlens, void *out,
                                       void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!a || !b || !cu_seqlens || !out) return MOE_EINVAL;
  if (G < 1 || G > kMaxG || M_total < 0 || Kd < 8 || N < 8 || Kd % 8 || N % 8) return MOE_EINVAL;
  if (op != MOE_GEMM_FWD && op != MOE_GEMM_DGRAD && op != MOE_GEMM_WGRAD) return MOE_EINVAL;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_EINVAL;
  if ((long long)M_total * (Kd > N ? Kd : N) >= (1LL << 40)) return MOE_EINVAL;
  // the operand loads address a 256-row tile of either operand with 32-bit byte offsets
  if (Kd > kMaxDim || N > kMaxDim) return MOE_EINVAL;
  // WGRAD's epilogue addresses a tile's fp32 rows with 32-bit buffer offsets (row * N * 4
  // plus an out-of-range marker for masked chunks), which must not wrap
  if (op == MOE_GEMM_WGRAD && N > (1 << 20)) return MOE_EINVAL;
  if (ws && ws_bytes < moe_group_gemm_workspace_bytes(op, dtype)) return MOE_ENOSPACE;
  if (M_total == 0) return MOE_OK;
  if (dtype == MOE_F32) {
    if (op == MOE_GEMM_WGRAD) {
      const long long n = (long long)G * Kd * N;
      hipLaunchKernelGGL(k_ggemm_f32_wgrad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                         stream, (const float *)a, (const float *)b, cu_seqlens, (float *)out, G,
                         M_total, Kd, N);
    } else {
      const long long n = (long long)M_total * (op == MOE_GEMM_FWD ? N : Kd);
      if (op == MOE_GEMM_FWD)
        hipLaunchKernelGGL(k_ggemm_f32_rows<MOE_GEMM_FWD>, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, stream, (const float *)a, (const float *)b, cu_seqlens,
                           (float *)out, G, M_total, Kd, N);
      else
        hipLaunchKernelGGL(k_ggemm_f32_rows<MOE_GEMM_DGRAD>, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, stream, (const float *)a, (const float *)b, cu_seqlens,
                           (float *)out, G, M_total, Kd, N);
    }
    return launch_status();
  }
  const uint16_t *a16 = (const uint16_t *)a, *b16 = (const uint16_t *)b;
  // FWD and DGRAD run 4 waves of 128x128, WGRAD 8 waves of 128x64 (its fp32
  // read-modify-write epilogue needs the registers); DGRAD loads 64-wide K stages.
  switch (op) {
    case MOE_GEMM_FWD:
      launch_rows<MOE_GEMM_FWD, 2>(Kd, a16, b16, cu_seqlens, out, nullptr, ws, G, M_total, Kd, N,
                                   stream);
      break;
    case MOE_GEMM_DGRAD:
      launch_rows<MOE_GEMM_DGRAD, 2>(N, a16, b16, cu_seqlens, out, nullptr, ws, G, M_total, Kd,
                                     N, stream);
      break;
    default:
      hipLaunchKernelGGL((k_ggemm_bf16<MOE_GEMM_WGRAD, false, 4>), dim3(device_cu_count()),
                         dim3(Waves<4>::threads), 0, stream, a16, b16, cu_seqlens, out, nullptr,
                         nullptr, G, M_total, Kd, N, GatherParams{});
  }
  return launch_status();
}

extern "C" moe_status_t moe_group_gemm_swiglu(moe_dtype dtype, int32_t G, int32_t M_total,
                                              int32_t Kd, int32_t N, const void *a,
                                              const void *b, const int32_t *cu_seqlens,
                                              void *z, void *h, void *ws, size_t ws_bytes,
                                              hipStream_t stream) {
  if (!a || !b || !cu_seqlens || !z) return MOE_EINVAL;
  if (dtype != MOE_BF16) return MOE_EINVAL;
  if (G < 1 || G > kMaxG || M_total < 0 || Kd < 8 || N < 16 || Kd % 8 || N % 16) return MOE_EINVAL;
  if ((long long)M_total * (Kd > N ? Kd : N) >= (1LL << 40)) return MOE_EINVAL;
  if (Kd > kMaxDim || N > kMaxDim) return MOE_EINVAL;
  if (ws && ws_bytes < moe_group_gemm_workspace_bytes(MOE_GEMM_FWD, dtype)) return MOE_ENOSPACE;
  if (M_total == 0) return MOE_OK;
  // 8 waves: the gated epilogue needs the registers the 128x128 wave tile would take
  launch_rows<kOpSwiglu, 4>(Kd, (const uint16_t *)a, (const uint16_t *)b, cu_seqlens, z, h, ws,
                            G, M_total, Kd, N, stream);
  return launch_status();
}

// floor(e / d) = mulhi(2 e, magic) >> shift = (e * magic) >> (31 + shift) for every
// 0 <= e < 2^31 and d >= 1: with shift = ceil(log2 d) and magic = floor(2^(31 + shift) / d) + 1
// (< 2^32), the product's error stays below one unit of the quotient for 31-bit dividends (the
// round-up method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  Doubling the dividend keeps the high word's shift non-negative, so
// d = 1 needs no special case.
static void div_magic(int32_t d, uint32_t *magic, int *shift) {
  int l = 0;
  while ((1LL << l) < d) ++l;
  *magic = (uint32_t)((1ULL << (31 + l)) / (unsigned long long)d + 1);
  *shift = l;
}

extern "C" moe_status_t moe_group_gemm_gather(moe_gemm_op op, moe_dtype dtype, int32_t G,
                                              int32_t M_total, int32_t Kd, int32_t N,
                                              const void *x_src, int64_t src_rows,
                                              const int32_t *gather, int32_t gather_div,
                                              const void *b, const int32_t *cu_seqlens,
                                              void *out, void *ws, size_t ws_bytes,
                                              hipStream_t stream) {
  if (!x_src || !gather || !b || !cu_seqlens || !out) return MOE_EINVAL;
  if (dtype != MOE_BF16 || (op != MOE_GEMM_FWD && op != MOE_GEMM_WGRAD)) return MOE_EINVAL;
  if (G < 1 || G > kMaxG || M_total < 0 || Kd < 8 || N < 8 || Kd % 8 || N % 8) return MOE_EINVAL;
  if (src_rows < 1 || src_rows >= (1LL << 31) || gather_div < 1) return MOE_EINVAL;
  if ((long long)M_total * (Kd > N ? Kd : N) >= (1LL << 40)) return MOE_EINVAL;
  if (Kd > kMaxDim || N > kMaxDim) return MOE_EINVAL;
  if (op == MOE_GEMM_WGRAD && N > (1 << 20)) return MOE_EINVAL;
  if (ws && ws_bytes < moe_group_gemm_workspace_bytes(op, dtype)) return MOE_ENOSPACE;
  if (M_total == 0) return MOE_OK;
  GatherParams gp;
  gp.x = (const char *)x_src;
  gp.ld_bytes = (uint32_t)Kd * 2;
  gp.idx = gather;
  gp.n_tok = (int)src_rows;
  gp.div = gather_div;
  div_magic(gather_div, &gp.magic, &gp.shift);
  const uint16_t *b16 = (const uint16_t *)b;
  if (op == MOE_GEMM_FWD)
    launch_rows<MOE_GEMM_FWD, 2, true>(Kd, nullptr, b16, cu_seqlens, out, nullptr, ws, G,
                                       M_total, Kd, N, stream, gp);
  else
    hipLaunchKernelGGL((k_ggemm_bf16<MOE_GEMM_WGRAD, false, 4, true>), dim3(device_cu_count()),
                       dim3(Waves<4>::threads), 0, stream, nullptr, b16, cu_seqlens, out,
                       nullptr, nullptr, G, M_total, Kd, N, gp);
  return launch_status();
}
