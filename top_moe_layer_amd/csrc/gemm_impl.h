// Grouped MFMA GEMM for the three FFN projections (gfx950, wave64).
//
// Every projection is nn.Linear(in, out, bias=False) applied to token rows
// (MiniMind lesson 13, section 3 step 3; section 0 equations): out = A W^T with
// A [rows, K] and W [Nout, K], both contiguous along K.  For the MoE each
// expert's rows form one group (the per-expert token lists of walkthrough
// step 5); the kernel walks a flattened list of (group, row-tile) x column-tile
// work items whose group boundaries it reads from the device-side expert
// offsets, so no host synchronisation is needed.
//
// Block: WM x WN wavefronts; block tile BM x BN of every output matrix (two
// matrices, gate and up, for the first projection).  K advances in slices of
// RB bytes per row (RB / sizeof(T) elements).  Slices are fetched straight
// into an S-deep LDS ring with global_load_lds_dwordx4 (no register staging),
// so up to S slices are in flight while the MFMAs consume the oldest one.
// LDS rows keep their 16-byte chunks at slot chunk ^ ((row / (256 / RB)) % CH)
// (CH chunks per row), which makes the 16-byte fragment reads bank-conflict
// free on the 64-bank LDS.  Arithmetic intensity against the L2 -> LDS
// traffic is BM*BN*NB / (BM + NB*BN) flop per byte, which is what bounds these
// kernels on MI355X; the 8-wavefront 256-row tiles double it over 4-wavefront
// 128-row tiles while keeping two wavefronts per SIMD.
// MFMA: v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32),
// fp32 accumulation.
//
// Epilogues:
//   gate/up : h = SiLU(g) * u = g * u / (1 + e^-g)  (lesson 13, section 1.2),
//             stored in the operand dtype in grouped row order;
//   down    : o * alpha_{t,j} (the router weight; 1 for the dense FFN),
//             written to y[t] (k == 1 or dense; plus the residual stream when
//             given, rounded once) or to the slot of entry (t, j) (k >= 2, in
//             the operand dtype) for the fixed-order combine.
//
// Decode-sized inference calls (the 64 x 128 tiles of eight wavefronts) can
// group the entries by expert in every block's prologue instead of reading
// the permutation kernel's lists (GemmParams::inl_*), and with at most one
// row tile of tokens and E <= 16 the gate/up launch takes every token against
// every expert while its last blocks run the router (GemmParams::allx_n,
// rt_*).
#pragma once

#include "device_common.h"
#include "kernels.h"
#include "router_impl.h"

namespace topmoe {

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  static constexpr int BK = 64;  // elements per 128-byte row chunk
  __device__ static __forceinline__ void mma(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// fp32: each 16-byte fragment holds 4 consecutive k of one lane group; the two
// lane groups (lanes 0-31, 32-63) cover k = 8q + s and 8q + 4 + s.  A and B use
// the same assignment, so the 4 depth-2 MFMAs sum all 8 k of the step.
template <>
struct Mfma<float> {
  static constexpr int BK = 32;
  __device__ static __forceinline__ void mma(f32x16& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c,
                                               0, 0, 0);
  }
};

// Scheduling hints for one MFMA region: spread NDS LDS operations (mask
// DSMASK: 0x100 reads, 0x200 writes) over the first MFMAs of the region and
// NVM global loads over all of them, so the memory pipes work while the MFMA
// pipe is busy instead of before or after it.
template <int I, int NMFMA, int NDS, int DSMASK, int NVM>
struct Interleave {
  __device__ static __forceinline__ void run() {
    if constexpr (I < NMFMA) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int spread = NMFMA > 1 ? (NMFMA + 1) / 2 : 1;  // LDS ops in the first half
      constexpr int ds = (I < spread) ? ((I + 1) * NDS / spread - I * NDS / spread) : 0;
      if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(DSMASK, ds, 0);
      constexpr int vm = (I + 1) * NVM / NMFMA - I * NVM / NMFMA;
      if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);
      Interleave<I + 1, NMFMA, NDS, DSMASK, NVM>::run();
    }
  }
};

// One 16-byte-per-lane direct-to-LDS load (global_load_lds_dwordx4): lane i
// writes lds + 16 i.  `lds` must be the same for every lane of the wavefront.
// (Kept out of the kernel template: called directly from the template, the
// target builtin suppresses the kernel's host launch stub.)
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// A pointer that is the same on every lane, moved to scalar registers so that
// base + 32-bit lane offset compiles to the saddr + voffset load form.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

// s_waitcnt with vmcnt(N) and the other counters left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for data written to LDS by direct-to-LDS loads: every
// wavefront first waits for its own loads (vmcnt) and its own LDS reads
// (lgkmcnt, so no read of a slot is outstanding when it is refilled), then
// s_barrier; the acquire fence keeps later LDS reads below the barrier.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 0xC00F);  // lgkmcnt(0), vm/exp at max
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Workgroup barrier for plain LDS stores: waits for this wavefront's LDS
// operations only (not for its direct-to-LDS loads in flight); the memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Operands and products of each kind: NA A matrices and NB B matrices share
// one LDS slice (A0, A1, B0, B1, B2 in that order); product p multiplies
// A pa(p) by B pb(p) into accumulator p.
template <int KIND>
struct KindTraits {  // the down projections
  static constexpr int NA = 1, NB = 1, NP = 1;
  static constexpr bool META = true, KGROUP = false, GATHER = false;
  __host__ __device__ static constexpr int pa(int) { return 0; }
  __host__ __device__ static constexpr int pb(int) { return 0; }
};
template <>
struct KindTraits<KIND_GATEUP> {  // x against Wg and Wu
  static constexpr int NA = 1, NB = 2, NP = 2;
  static constexpr bool META = false, KGROUP = false, GATHER = true;
  __host__ __device__ static constexpr int pa(int) { return 0; }
  __host__ __device__ static constexpr int pb(int q) { return q; }
};
template <>
struct KindTraits<KIND_BWD_GU> {  // x against Wg and Wu (recomputed for the backward)
  static constexpr int NA = 1, NB = 2, NP = 2;
  static constexpr bool META = false, KGROUP = false, GATHER = true;
  __host__ __device__ static constexpr int pa(int) { return 0; }
  __host__ __device__ static constexpr int pb(int q) { return q; }
};
template <>
struct KindTraits<KIND_BWD_DH> {  // dy against Wd^T
  static constexpr int NA = 1, NB = 1, NP = 1;
  static constexpr bool META = true, KGROUP = false, GATHER = true;
  __host__ __device__ static constexpr int pa(int) { return 0; }
  __host__ __device__ static constexpr int pb(int) { return 0; }
};
template <>
struct KindTraits<KIND_WGRAD2> {  // dg^T and du^T against x^T
  static constexpr int NA = 2, NB = 1, NP = 2;
  static constexpr bool META = false, KGROUP = true, GATHER = false;
  __host__ __device__ static constexpr int pa(int q) { return q; }
  __host__ __device__ static constexpr int pb(int) { return 0; }
};
template <>
struct KindTraits<KIND_WGRAD1> {  // (alpha dy)^T against h^T
  static constexpr int NA = 1, NB = 1, NP = 1;
  static constexpr bool META = false, KGROUP = true, GATHER = false;
  __host__ __device__ static constexpr int pa(int) { return 0; }
  __host__ __device__ static constexpr int pb(int) { return 0; }
};

template <typename T, int BM, int BN, int WM, int WN, int RB, int S, int KIND>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmParams p) {
  using KT_ = KindTraits<KIND>;
  constexpr int NA = KT_::NA, NB = KT_::NB, NP = KT_::NP;
  constexpr bool META = KT_::META;      // per-row entry / alpha in the epilogue
  constexpr bool KGROUP = KT_::KGROUP;  // groups along K (weight gradients)
  // split K (the down projection): each work item is one K chunk of a tile
  constexpr bool SPLIT = KIND == KIND_DOWN_PARTIAL;
  constexpr bool PAD = KGROUP || KIND == KIND_BWD_GU || KIND == KIND_BWD_DH;  // padded group columns
  constexpr int NW = WM * WN;                // wavefronts: WM along rows x WN along columns
  constexpr int NTHR = 64 * NW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wavefront and matrix
  constexpr int R = NA * BM + NB * BN;       // LDS rows per slice: A0 (, A1), B0 (, B1, B2)
  constexpr int A_BYTES = NA * BM * RB, B_BYTES = BN * RB;
  constexpr int STAGE = R * RB;
  constexpr int CH = RB / 16;                // 16-byte chunks per LDS row
  constexpr int RPW = 256 / RB;              // rows per 256-byte bank window
  constexpr int RPI = 1024 / RB;             // rows per 1 KB direct-to-LDS load
  constexpr int LPW = R / RPI / NW;          // direct-to-LDS loads per wavefront per slice
  constexpr int QS = RB / 32;                // MFMA sub-steps per slice
  constexpr int EPS = RB / int(sizeof(T));   // K elements per slice
  static_assert(RB == 64 || RB == 128, "row bytes");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
  static_assert((R / RPI) % NW == 0 && LPW >= 1, "slice rows must split evenly over wavefronts");
  static_assert(BM % RPI == 0 && BN % RPI == 0, "a load stays in one operand");
  static_assert(S >= 2 && S * STAGE <= 156 * 1024, "LDS ring exceeds 156 KB");
  static_assert(BM % (16 / int(sizeof(T))) == 0, "staged rows split into 16-byte pieces");
  static_assert((S - 1) * LPW < 64, "vmcnt range");
  static_assert(BM <= NTHR, "one thread per tile row for the epilogue metadata");
  static_assert(!PAD || BM % 64 == 0, "padded groups end inside a group's last row tile");
  // One __shared__ object per ring slot: the compiler then sees that LDS reads
  // of one slot never alias direct-to-LDS loads into another and does not
  // drain the load queue before each read.
  __shared__ __attribute__((aligned(1024))) char ring0[STAGE];
  __shared__ __attribute__((aligned(1024))) char ring1[STAGE];
  __shared__ __attribute__((aligned(1024))) char ring2[S > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char ring3[S > 3 ? STAGE : 16];
  __shared__ int s_scan[64];
  __shared__ int s_off[65];
  __shared__ int s_poff[PAD ? 64 : 1];
  __shared__ int s_ment[META ? BM : 1];
  __shared__ float s_malpha[META ? BM : 1];
  __shared__ float s_dal[KIND == KIND_BWD_DH ? WN * BM : 1];
  // backward: a transposed output tile [BN][BM + 16 bytes] on its way out,
  // where it fits beside the ring (else the transposed stores go direct)
  constexpr int LDST = BM + 16 / int(sizeof(T));
  constexpr bool STAGE_T = (KIND == KIND_BWD_GU || KIND == KIND_BWD_DH) &&
                           S * STAGE + BN * LDST * int(sizeof(T)) <= 156 * 1024;
  __shared__ __attribute__((aligned(16))) T s_stage[STAGE_T ? BN * LDST : 1];
  // Row-major outputs go out four columns per store after a transpose inside
  // each lane quad -- except from gate/up tiles whose two accumulator sets
  // already hold half of a wavefront's 256 registers at two wavefronts per
  // SIMD: there the transpose's temporaries would spill, so they store
  // element by element.
  constexpr bool QT =
      !((KIND == KIND_GATEUP || KIND == KIND_BWD_GU) && NP * TM * TN * 16 >= 128 && NW == 8);

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the router blocks of a decode gate/up launch (LDS: the ring, unused here)
  if constexpr (KIND == KIND_GATEUP && BM == 64 && BN == 128 && NTHR >= kInlineMaxEntries) {
    if (p.rt_blocks > 0 && int(blockIdx.x) >= int(gridDim.x) - p.rt_blocks) {
      int* s_rcnt = reinterpret_cast<int*>(ring0);
      float(*s_rpart)[64] = reinterpret_cast<float(*)[64]>(ring0 + 256);
      float(*s_rps)[64] = reinterpret_cast<float(*)[64]>(ring0 + 256 + 1024);
      rt::route_split_block_upto16<T>(static_cast<const T*>(p.A), p.rt_wr, p.rt_n, p.K, p.E, p.k,
                                      p.rt_renorm != 0, p.rt_tb,
                                      int(blockIdx.x) - (int(gridDim.x) - p.rt_blocks),
                                      p.rt_blocks, p.rt_topk, p.rt_alpha, p.rt_count, p.rt_psum,
                                      p.rt_zpart, s_rcnt, s_rpart, s_rps);
      return;
    }
  }
  const int nt_count = (p.Nout + BN - 1) / BN;
  const int KTu = KGROUP ? 0 : p.K / EPS;  // K slices of every tile (row-grouped kinds)
  const int64_t rowbytes = int64_t(p.K) * int64_t(sizeof(T));  // A and B row pitch

  // ---- groups: per-group row offsets and tile counts from the device-side
  // offsets (or one group), and with PAD the padded offsets: each group's
  // rows rounded up to 64, which is where they sit in the transposed
  // (K-major) activations of the weight gradients.  Cached in LDS.
  // In-block routing (GemmParams::inl_topk): only the decode-sized forward
  // tiles (64 x 128, one thread per entry) carry it.
  constexpr bool INL = !KGROUP && !PAD && BM == 64 && BN == 128 && NTHR >= kInlineMaxEntries &&
                       (KIND == KIND_GATEUP || KIND == KIND_DOWN_Y || KIND == KIND_DOWN_SLOTS);
  constexpr int IMAX = INL ? kInlineMaxEntries : 1;
  __shared__ int s_ient[IMAX];       // grouped row -> entry id (t*k + j)
  __shared__ float s_ialpha[IMAX];   // grouped row -> alpha
  __shared__ int s_icnt[INL ? 64 : 1];
  __shared__ int s_iw[INL ? NW * 64 : 1];
  __shared__ double s_ips[INL ? 64 : 1];
  const bool inl = INL && p.inl_topk != nullptr;
  const bool allx = INL && p.allx_n > 0;  // every token against every expert
  const bool grouped = p.offsets != nullptr || inl || allx;
  const int G = grouped ? p.E : 1;
  // the extra block of an in-block-routed launch (routing outputs only)
  const bool outs_block = INL && inl && p.inl_outputs != 0 && blockIdx.x == gridDim.x - 1;
  if constexpr (INL) {
    if (inl) {
      // The entries (t*k + j order, one per thread) grouped by expert as the
      // permutation kernel groups them.  Each wavefront counts its entries per
      // expert with ballots (an entry's rank among its wavefront's entries of
      // the same expert: the matching lanes below it); wavefront 0 turns the
      // counts into per-wavefront prefixes, expert totals and exclusive
      // offsets; each entry then lands at offset + earlier wavefronts' count
      // + rank in its wavefront.
      const int e = tid < p.inl_n ? p.inl_topk[tid] : -1;
      const float a = (META && tid < p.inl_n) ? p.inl_alpha[tid] : 0.f;
      const bool valid = e >= 0;
      // this wavefront's row of counts: cleared and written by the wavefront
      // itself (its LDS operations complete in order)
      s_iw[wid * 64 + lane] = 0;
      uint64_t peers = 0ull;
      uint64_t todo = __ballot(valid);
      while (todo) {
        const int leader = __ffsll((long long)todo) - 1;
        const int le = __builtin_amdgcn_readlane(e, leader);  // scalar: no LDS round trip
        const uint64_t m = __ballot(valid && e == le);
        if (valid && e == le) peers = m;
        todo &= ~m;
      }
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      const int in_wave = __popcll(peers & below);
      if (valid && in_wave == 0) s_iw[wid * 64 + e] = __popcll(peers);
      __syncthreads();
      if (tid < 64) {  // lane = expert
        int run = 0;
        for (int w = 0; w < NW; ++w) {
          const int c = s_iw[w * 64 + lane];
          s_iw[w * 64 + lane] = run;
          run += c;
        }
        const int c = lane < G ? run : 0;
        // one scan for the entries (low half) and the row tiles (high half):
        // at most 512 entries and 72 tiles, so neither half carries over
        const int both = wave_inclusive_scan(c | (((c + BM - 1) / BM) << 16), lane);
        const int incl = both & 0xffff;
        if (lane < G) s_off[lane] = incl - c;
        if (lane == G - 1) s_off[G] = incl;
        s_scan[lane] = both >> 16;
        s_icnt[lane] = c;
      }
      __syncthreads();
      if (valid) {
        const int d = s_off[e] + s_iw[wid * 64 + e] + in_wave;
        s_ient[d] = tid;
        s_ialpha[d] = a;
      }
      __syncthreads();
      if (outs_block) {
        // The routing outputs of the permutation kernel.  aux = E * coef *
        // sum_e c_e * (sum_t p_{t,e}) / N^2 and z = z_coef * sum lse^2 / N:
        // fp64 sums in the permutation kernel's order (per expert, lanes
        // stride over the router blocks, then a wavefront sum; then the
        // wavefront sum of the c_e terms), so both paths give the same bits.
        if (p.inl_offsets_out != nullptr && tid <= G) p.inl_offsets_out[tid] = s_off[tid];
        if (p.inl_sorted_out != nullptr)
          for (int d = tid; d < p.inl_n; d += NTHR) p.inl_sorted_out[d] = s_ient[d] / p.k;
        const int nb = p.inl_nblk;
        const double n = double(p.inl_tokens);
        const bool aux = p.inl_aux_out != nullptr && p.inl_psum_part != nullptr;
        if (aux) {
          for (int g = wid; g < G; g += NW) {
            double ps = 0.0;
            for (int b = lane; b < nb; b += 64) ps += double(p.inl_psum_part[int64_t(g) * nb + b]);
            ps = wave_sum(ps);
            if (lane == 0) s_ips[g] = ps;
          }
        }
        if (wid == NW - 1 && p.inl_z_out != nullptr && p.inl_z_part != nullptr) {
          double z = 0.0;
          for (int b = lane; b < nb; b += 64) z += double(p.inl_z_part[b]);
          z = wave_sum(z);
          if (lane == 0)
            *p.inl_z_out = (p.inl_z_coef != 0.f && n > 0) ? float(double(p.inl_z_coef) * z / n) : 0.f;
        }
        __syncthreads();
        if (aux && wid == 0) {
          const double term = wave_sum(lane < G ? double(s_icnt[lane]) * s_ips[lane] : 0.0);
          if (lane == 0)
            *p.inl_aux_out = (p.inl_coef != 0.f && n > 0) ?
                float(double(p.E) * double(p.inl_coef) * term / (n * n)) : 0.f;
        }
        return;
      }
    }
  }
  if (allx && !inl) {  // E groups of the N rows of A, in order
    if (tid < 64) {
      const int n = int(p.allx_n), mt = (n + BM - 1) / BM;
      if (lane <= G) s_off[lane] = lane * n;
      s_scan[lane] = (lane < G ? lane + 1 : G) * mt;
    }
    __syncthreads();
  } else if (!inl && (p.offsets != nullptr || PAD)) {
    if (tid < 64) {
      int c = 0;
      if (lane < G) {
        const int dense_rows = KGROUP ? int(p.kcount) : int(p.M);
        const int o0 = p.offsets != nullptr ? p.offsets[lane] : 0;
        const int o1 = p.offsets != nullptr ? p.offsets[lane + 1] : dense_rows;
        c = o1 - o0;
        s_off[lane] = o0;
        if (lane == G - 1) s_off[G] = o1;
      }
      const int tiles = (c + BM - 1) / BM;
      s_scan[lane] = wave_inclusive_scan(tiles, lane);
      if constexpr (PAD) {
        const int kp = (c + 63) & ~63;
        const int incl = wave_inclusive_scan(kp, lane);
        if (lane < G) s_poff[lane] = incl - kp;
      }
    }
    __syncthreads();
  }

  struct Tile {
    int e, rows, n0, kt, koff, chunk;
    int64_t row0;
  };
  // ---- work list.
  // Row-grouped kinds: persistent and XCD-aware.  Blocks are dispatched to
  // the 8 XCDs round robin (block b runs on XCD b % 8), each XCD with its own
  // L2.  XCD x owns the contiguous range [x*per, (x+1)*per) of the real
  // tiles, ordered in groups of GM M-tiles (column by column inside a group),
  // so co-resident blocks share A rows and weight panels in that L2; its
  // gridDim/8 blocks take the range round robin.
  // K-grouped kinds: one tile per block.  Every group has the same output
  // tiles; XCD x takes the x-th eighth of each group's tiles (so groups of
  // very different K spread evenly over the XCDs), groups in order.
  // M tiles per walk group: 8, and 4 for the down projections (measured on
  // the dense 16384 x 2048 x 6464 FFN: its down projection 2 % faster with
  // 4, its gate/up projection 0.5 % slower)
  constexpr int GM = (KIND == KIND_DOWN_Y || KIND == KIND_DOWN_SLOTS) ? 4 : 8;
  int total_mt = 0, total = 0, per = 0, nbx = 1, lb = 0, xbase = 0, n_my = 0;
  int kg_e = 0, kg_idx = 0, kg_mt = 0;
  if constexpr (KGROUP) {
    kg_mt = int((p.M + BM - 1) / BM);
    const int te = kg_mt * nt_count;
    const int c = (te + 7) >> 3;
    const int j = int(blockIdx.x >> 3);
    kg_e = j / c;
    kg_idx = int(blockIdx.x & 7) * c + (j - kg_e * c);
    n_my = (kg_e < G && kg_idx < te) ? 1 : 0;
  } else {
    total_mt = !grouped ? int((p.M + BM - 1) / BM)
                        : __builtin_amdgcn_readfirstlane(s_scan[p.E - 1]);
    total = total_mt * nt_count * (SPLIT ? p.ksplit : 1);
    per = (total + 7) >> 3;
    const int extra = (INL && inl && p.inl_outputs != 0 ? 1 : 0) +
                      (KIND == KIND_GATEUP && p.rt_blocks > 0 ? p.rt_blocks : 0);
    nbx = int((gridDim.x - extra) >> 3);
    lb = int(blockIdx.x >> 3);
    xbase = int(blockIdx.x & 7) * per;
    for (int l = lb; l < per && xbase + l < total; l += nbx) ++n_my;
  }
  if (n_my == 0) return;

  auto decode = [&](int j) -> Tile {
    Tile t;
    if constexpr (KGROUP) {
      const int first_m = (kg_idx / (GM * nt_count)) * GM;
      const int gsz = min(kg_mt - first_m, GM);
      const int in_group = kg_idx - first_m * nt_count;
      const int mt = first_m + in_group % gsz;
      t.n0 = (in_group / gsz) * BN;
      t.e = kg_e;
      t.row0 = int64_t(mt) * BM;
      const int64_t left = p.M - t.row0;
      t.rows = left < BM ? int(left) : BM;
      const int c = s_off[kg_e + 1] - s_off[kg_e];
      t.kt = ((c + 63) & ~63) / EPS;
      t.koff = s_poff[kg_e];
      t.chunk = 0;
    } else {
      int L = xbase + lb + j * nbx;
      t.chunk = 0;
      if constexpr (SPLIT) {  // chunk-major: the tiles of one K chunk, then the next chunk's
        const int tiles = total_mt * nt_count;
        t.chunk = L / tiles;
        L -= t.chunk * tiles;
      }
      const int first_m = (L / (GM * nt_count)) * GM;
      const int gsz = min(total_mt - first_m, GM);
      const int in_group = L - first_m * nt_count;
      const int mt = first_m + in_group % gsz;
      t.n0 = (in_group / gsz) * BN;
      t.kt = KTu;
      t.koff = 0;
      if constexpr (SPLIT) {  // the chunk's slices (every chunk holds at least one)
        const int k0 = t.chunk * p.kchunk;
        t.kt = min(p.kchunk, KTu - k0);
        t.koff = k0 * EPS;
      }
      if (!grouped) {
        t.e = 0;
        t.row0 = int64_t(mt) * BM;
        const int64_t left = p.M - t.row0;
        t.rows = left < BM ? int(left) : BM;
      } else {
        int ge = 0;  // group = number of groups whose tiles all precede mt
        for (int g = 0; g < p.E; ++g) ge += (s_scan[g] <= mt) ? 1 : 0;
        const int local_t = mt - (ge > 0 ? s_scan[ge - 1] : 0);
        t.e = ge;
        t.row0 = s_off[ge] + int64_t(local_t) * BM;
        const int left = s_off[ge + 1] - int(t.row0);
        t.rows = left < BM ? left : BM;
      }
    }
    // uniform over the block: keep the tile in scalar registers
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.kt = __builtin_amdgcn_readfirstlane(t.kt);
    t.koff = __builtin_amdgcn_readfirstlane(t.koff);
    if constexpr (SPLIT) t.chunk = __builtin_amdgcn_readfirstlane(t.chunk);
    t.row0 = __builtin_amdgcn_readfirstlane(int(t.row0));
    return t;
  };

  // ---- direct-to-LDS load sources.  Wavefront w fills LDS row blocks
  // w*LPW .. w*LPW+LPW-1 (RPI rows = 1 KB each) of every slice.  Lane i of a
  // load writes slot base + 16 i, i.e. row RPI*b + i/CH, slot i%CH; it
  // therefore fetches logical chunk (i%CH) ^ swizzle(row).  Rows past the
  // tile's valid rows / columns are clamped to the last valid one (in bounds,
  // results discarded).  A-row indices of a tile are fetched early (`rid`)
  // and turned into addresses only when that tile's first slice is issued.
  auto load_rows = [&](const Tile& t, int32_t(&rid)[LPW]) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int r = (wid * LPW + j) * RPI + lane / CH;
      const bool is_a = r < NA * BM;
      const int lr = (NA == 2 && r >= BM) ? r - BM : r;
      int gr = int(t.row0) + (lr < t.rows ? lr : t.rows - 1);
      if (!is_a) gr = 0;
      int ent = gr;
      if constexpr (INL) {
        if (inl) ent = s_ient[gr];
      }
      if (!inl && p.entries != nullptr) ent = p.entries[gr];
      int row = (KT_::GATHER && is_a && (inl || p.entries != nullptr)) ? ent / p.k : gr;
      if constexpr (INL) {
        // every token against every expert: gate/up reads token gr - e N;
        // the down projection reads entry (t, j)'s row e N + t
        if (allx && is_a)
          row = inl ? int(t.e) * int(p.allx_n) + ent / p.k : gr - int(t.e) * int(p.allx_n);
      }
      rid[j] = row;
    }
  };
  int32_t rid[LPW];          // A-row indices of the next tile
  const char* sbase[LPW];    // per-load base pointers (uniform) of the tile being issued
  uint32_t voff[LPW];        // per-lane byte offsets from them
  // Load j of a wavefront covers RPI consecutive LDS rows, all in one of the
  // A0, A1, B0, B1, B2 regions (BM, BN are multiples of RPI), so its base
  // pointer is uniform (scalar registers) and each lane keeps only a 32-bit
  // byte offset (the global_load_lds saddr + voffset form).  Operand
  // matrices are below 4 GiB (activations as a whole, each expert's weight
  // matrix on its own).
  auto make_src = [&](const Tile& t, const int32_t(&rid)[LPW]) {
    const int64_t kbytes = int64_t(t.koff) * int64_t(sizeof(T));  // K-grouped: the group's columns
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int r0 = (wid * LPW + j) * RPI;  // first row of the load (uniform)
      const int r = r0 + lane / CH;
      const int chunk = (lane % CH) ^ ((r / RPW) % CH);
      if (r0 < NA * BM) {
        const char* a = static_cast<const char*>((NA == 2 && r0 >= BM) ? p.A1 : p.A);
        sbase[j] = a + kbytes;
        voff[j] = uint32_t(rid[j]) * uint32_t(rowbytes) + uint32_t(chunk * 16);
      } else {
        const int rb = r - NA * BM;
        const int which = (r0 - NA * BM) / BN;  // uniform
        int n = t.n0 + rb - which * BN;
        n = n < p.Nout ? n : p.Nout - 1;
        const void* b = which == 0 ? p.B0 : (NB > 1 && which == 1) ? p.B1 : p.B2;
        sbase[j] = static_cast<const char*>(b) +
                   (KGROUP ? kbytes
                           : int64_t(t.e) * p.Nout * rowbytes + (SPLIT ? kbytes : int64_t(0)));
        voff[j] = uint32_t(n) * uint32_t(rowbytes) + uint32_t(chunk * 16);
      }
    }
  };
  auto slot_ptr = [&](int slot) -> char* {
    return slot == 0 ? ring0 : slot == 1 ? ring1 : slot == 2 ? ring2 : ring3;
  };
  auto issue = [&](int kt, char* slot_base) {
    const uint32_t ko = uint32_t(kt) * RB;
    char* dst = slot_base + wid * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      lds_dma16(uniform_ptr(sbase[j]) + uint64_t(voff[j] + ko), dst + j * 1024);
  };

  f32x16 acc[NP][TM][TN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int b = 0; b < NP; ++b)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.f;
  };

  const int fr = lane & 31, fg = lane >> 5;
  const int wm = (wid / WN) * WTM, wn = (wid % WN) * WTN;
  const int sw = (fr / RPW) % CH;  // row swizzle (32-row fragment blocks keep it)

  // MFMA operand fragments, double-buffered in registers: the fragments of
  // sub-step q + 1 are read from LDS while the MFMAs of sub-step q run.
  u32x4 fa0[NA][TM], fb0[NB][TN], fa1[NA][TM], fb1[NB][TN];
  auto frag_load = [&](const char* sb, int q, u32x4(&fa)[NA][TM], u32x4(&fb)[NB][TN]) {
    const int rd = ((2 * q + fg) ^ sw) << 4;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[a][i] = *reinterpret_cast<const u32x4*>(sb + (a * BM + wm + 32 * i + fr) * RB + rd);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[b][j] = *reinterpret_cast<const u32x4*>(sb + A_BYTES + b * B_BYTES +
                                                   (wn + 32 * j + fr) * RB + rd);
  };
  auto mma_all = [&](const u32x4(&fa)[NA][TM], const u32x4(&fb)[NB][TN]) {
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          Mfma<T>::mma(acc[q][i][j], fa[KT_::pa(q)][i], fb[KT_::pb(q)][j]);
  };

  constexpr int MF = NP * TM * TN * (sizeof(T) == 4 ? 4 : 1);  // MFMAs per sub-step
  constexpr int DSR = NA * TM + NB * TN;                       // LDS reads per sub-step

  // One K slice (QS MFMA sub-steps of 16 k), reading slot `cur`:
  //   LDS reads of sub-step q+1 | MFMAs of sub-step q   (q < QS - 1)
  //   wait for the next slice, barrier, refill `cur` (see `what`)
  //   LDS reads of the next slice's sub-step 0 (slot `nxt`) | MFMAs of the last sub-step
  // `full_wait`: the next slice is the last one in flight, so drain everything.
  auto step = [&](char* cur, char* nxt, bool full_wait, bool refill, int ikt) {
    __builtin_amdgcn_sched_barrier(0);
    frag_load(cur, 1, fa1, fb1);
    mma_all(fa0, fb0);
    Interleave<0, MF, DSR, 0x100, 0>::run();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QS == 4) {
      frag_load(cur, 2, fa0, fb0);
      mma_all(fa1, fb1);
      Interleave<0, MF, DSR, 0x100, 0>::run();
      __builtin_amdgcn_sched_barrier(0);
      frag_load(cur, 3, fa1, fb1);
      mma_all(fa0, fb0);
      Interleave<0, MF, DSR, 0x100, 0>::run();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (full_wait) wait_vmcnt<0>();
    else wait_vmcnt<(S - 2) * LPW>();
    ring_barrier();
    if (refill) issue(ikt, cur);
    __builtin_amdgcn_sched_barrier(0);
    frag_load(nxt, 0, fa0, fb0);
    mma_all(fa1, fb1);
    Interleave<0, MF, DSR, 0x100, 0>::run();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- epilogue.  32x32 accumulator layout: lane (fr, fg), register v holds
  // row 8*(v/4) + 4*fg + v%4, column fr of the MFMA tile.
  int m_ent = 0;
  float m_alpha = 1.f;
  auto load_meta = [&](const Tile& t) {  // one row per thread, ahead of the epilogue
    if (META && tid < BM) {
      const int64_t g = t.row0 + (tid < t.rows ? tid : t.rows - 1);
      m_ent = p.entries != nullptr ? p.entries[g] : int(g);
      m_alpha = p.alpha != nullptr ? p.alpha[g] : 1.f;
      if constexpr (INL) {
        if (inl) {
          m_ent = s_ient[g];
          m_alpha = s_ialpha[g];
        }
      }
    }
  };
  // dh kind: the tile's (g, u) pairs, fetched with the metadata so that their
  // latency hides behind the tile's last K steps (zeros outside the tile).
  constexpr bool DHK = KIND == KIND_BWD_DH;
  typedef typename PairWord<T>::type pair_t;
  pair_t gu_pre[DHK ? TM : 1][DHK ? 16 : 1][DHK ? TN : 1];
  auto load_gu = [&](const Tile& t) {
    if constexpr (DHK) {
      int rl = wm + 4 * fg, cl = wn + fr;
      asm volatile("" : "+v"(rl), "+v"(cl));
      const int rows_left = t.rows - rl;
      const int cols_left = p.Nout - (t.n0 + cl);
      const pair_t* src = static_cast<const pair_t*>(p.gu);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ro = 32 * i + 8 * (v >> 2) + (v & 3);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const bool ok = ro < rows_left && 32 * j < cols_left;
            const int64_t e_idx = (t.row0 + rl + ro) * int64_t(p.Nout) + t.n0 + cl + 32 * j;
            gu_pre[i][v][j] = ok ? src[e_idx] : PairWord<T>::zero();
          }
        }
    }
  };
  auto epilogue = [&](const Tile& t) {
    if constexpr (META) {
      // The previous tile's reads of s_ment / s_malpha finished before the
      // ring barriers of this tile's steps (each drains this wavefront's LDS
      // operations first), so the rows can be overwritten here.
      if (tid < BM) { s_ment[tid] = m_ent; s_malpha[tid] = m_alpha; }
      lds_barrier();
    }
    // The lane's first row / column in the tile, made opaque so that the
    // per-register row numbers are not hoisted out of the tile loop (they
    // would hold dozens of registers for the whole block).
    int rl = wm + 4 * fg, cl = wn + fr;
    asm volatile("" : "+v"(rl), "+v"(cl));
    const int rows_left = t.rows - rl;            // valid: 32 i + 8 (v / 4) + v % 4 < rows_left
    const int cols_left = p.Nout - (t.n0 + cl);   // valid: 32 j < cols_left
    if constexpr (KIND == KIND_BWD_GU || KIND == KIND_BWD_DH) {
      // Backward epilogues, per element (column i of the intermediate, row t):
      //   gu: g, u (the accumulators) go out as a pair in the dtype, row-major;
      //       h = SiLU(g) u transposed into the group's padded columns (and,
      //       for the training forward, row-major into out2 as well).
      //   dh: with g, u read back, s = sigma(g), SiLU(g) = g s and
      //       SiLU'(g) = s (1 + g (1 - s)):  dh = alpha dh_raw,
      //       dg = dh u SiLU'(g),  du = dh SiLU(g);  [dg | du] row-major (the dx
      //       GEMM's A operand), dg and du transposed (the weight-gradient
      //       GEMMs' operands); d alpha gets dh_raw . h summed over the row.
      // Transposed outputs hold zeros in the group's padding rows.
      constexpr bool DH = KIND == KIND_BWD_DH;
      const int lr0 = int(t.row0) - s_off[t.e];  // tile start within its group
      const int64_t pcol0 = int64_t(s_poff[t.e]) + lr0;  // its first padded column
      const int kpad = ((s_off[t.e + 1] - s_off[t.e]) + 63) & ~63;
      const int pad_rows = kpad - lr0 < BM ? kpad - lr0 : BM;  // tile rows inside the padded group
      const int pad_left = pad_rows - rl;
      const int64_t ldk = p.ldk;
      // Transposed outputs: staged in LDS where it fits (each lane writes its
      // four consecutive rows of a column as one 8-byte word, then the block
      // copies whole 16-byte row pieces of consecutive tokens out); else
      // written directly, four rows per lane.
      auto copy_out = [&](T* dst) {
        constexpr int V = 16 / int(sizeof(T));
        constexpr int CPR = BM / V;
        for (int idx = tid; idx < BN * CPR; idx += NTHR) {
          const int c = idx / CPR, r = (idx - c * CPR) * V;
          if (t.n0 + c < p.Nout && r < pad_rows)
            *reinterpret_cast<u32x4*>(dst + int64_t(t.n0 + c) * ldk + pcol0 + r) =
                *reinterpret_cast<const u32x4*>(s_stage + c * LDST + r);
        }
      };
      auto put_t = [&](T* dst, int i, int vq, int j, const float (&v)[4]) {
        const int ro0 = 32 * i + 8 * vq;
        if constexpr (STAGE_T) {
          store4<T>(s_stage + (cl + 32 * j) * LDST + rl + ro0, v);
        } else {
          if (32 * j < cols_left && ro0 < pad_left)
            store4<T>(dst + int64_t(t.n0 + cl + 32 * j) * ldk + pcol0 + rl + ro0, v);
        }
      };
      const int q4 = fr & 3;
      const int cq = t.n0 + (cl & ~3);  // first column of the lane's quad
      float dal[DH ? TM * 16 : 1];
      float dus[DH ? TM : 1][DH ? 4 : 1][DH ? TN : 1][4];
#pragma unroll
      for (int n = 0; n < (DH ? TM * 16 : 1); ++n) dal[n] = 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const int ro0 = 32 * i + 8 * vq;
          const bool row_ok_t = ro0 + q4 < rows_left;  // the lane's row after the transpose
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const bool col_ok = 32 * j < cols_left;   // the same for the whole quad
            const int64_t rowbase = (t.row0 + rl + ro0 + q4) * int64_t(p.Nout) + cq + 32 * j;
            float t0[4];
            if constexpr (!DH) {
              float g4[4], u4[4];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const int v = 4 * vq + w;
                const bool ok = ro0 + w < rows_left && col_ok;
                g4[w] = acc[0][i][j][v];
                u4[w] = acc[1][i][j][v];
                t0[w] = ok ? silu_mul(g4[w], u4[w]) : 0.f;
              }
              if constexpr (QT) {
                quad_transpose(g4, q4);
                quad_transpose(u4, q4);
                if (row_ok_t && col_ok) store_pairs4<T>(p.out, rowbase, g4, u4);
                if (p.out2 != nullptr) {  // the forward's h as well, row-major
                  float h4[4] = {t0[0], t0[1], t0[2], t0[3]};
                  quad_transpose(h4, q4);
                  if (row_ok_t && col_ok) store4<T>(static_cast<T*>(p.out2) + rowbase, h4);
                }
              } else {
#pragma unroll
                for (int w = 0; w < 4; ++w)
                  if (ro0 + w < rows_left && col_ok) {
                    const int64_t o = (t.row0 + rl + ro0 + w) * int64_t(p.Nout) + t.n0 + cl + 32 * j;
                    store_pair<T>(p.out, o, g4[w], u4[w]);
                    if (p.out2 != nullptr) static_cast<T*>(p.out2)[o] = from_f32<T>(t0[w]);
                  }
              }
            } else {
              float dg4[4], du4[4];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const int v = 4 * vq + w;
                const bool ok = ro0 + w < rows_left && col_ok;
                float g, u;
                PairWord<T>::unpack(gu_pre[i][v][j], g, u);
                const float d = acc[0][i][j][v];
                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
                const float si = g * sg;
                const float dh = d * s_malpha[rl + ro0 + w];
                dg4[w] = dh * u * (sg * (1.0f + g * (1.0f - sg)));
                du4[w] = dh * si;
                dal[16 * i + v] += d * (si * u);  // zero where not ok (g = u = 0)
                t0[w] = ok ? dg4[w] : 0.f;
                dus[i][vq][j][w] = ok ? du4[w] : 0.f;
              }
              quad_transpose(dg4, q4);
              quad_transpose(du4, q4);
              if (row_ok_t && col_ok) {
                T* o = static_cast<T*>(p.out) + (t.row0 + rl + ro0 + q4) * (2 * int64_t(p.Nout)) +
                       cq + 32 * j;
                store4<T>(o, dg4);
                store4<T>(o + p.Nout, du4);
              }
            }
            put_t(static_cast<T*>(p.out1), i, vq, j, t0);
          }
        }
      }
      if constexpr (STAGE_T) {
        lds_barrier();
        copy_out(static_cast<T*>(p.out1));
      }
      if constexpr (DH) {
        if constexpr (STAGE_T) lds_barrier();  // every piece of dg^T has been read
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int vq = 0; vq < 4; ++vq)
#pragma unroll
            for (int j = 0; j < TN; ++j) put_t(static_cast<T*>(p.out2), i, vq, j, dus[i][vq][j]);
        if constexpr (STAGE_T) {
          lds_barrier();
          copy_out(static_cast<T*>(p.out2));
        }
      }
      if constexpr (DH) {
        if (p.dalpha_part != nullptr) {
          // Row sums over the wavefront's columns (the 32 lanes fr of each
          // half-wavefront), then over the WN wavefronts.  Halving exchanges:
          // at mask m a lane with (fr & m) keeps the upper half of its values
          // and adds its partner's; once one value is left, plain butterflies.
          // Lane fr ends with the sum for value index fr >> (5 - STEPS).
          constexpr int V = TM * 16;
          constexpr int STEPS = V >= 32 ? 5 : 4;  // TM >= 1: V is 16, 32 or more
          constexpr int CNT = V >> STEPS;
#pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            const int mask = 16 >> st;
            const int half = V >> (st + 1);
            const bool upper = (fr & mask) != 0;
#pragma unroll
            for (int n = 0; n < half; ++n) {
              const float send = upper ? dal[n] : dal[n + half];
              const float keep = upper ? dal[n + half] : dal[n];
              dal[n] = keep + __shfl_xor(send, mask, 64);
            }
          }
          if constexpr (STEPS < 5) dal[0] += __shfl_xor(dal[0], 1, 64);
          constexpr int sh = 5 - STEPS;
          if ((fr & ((1 << sh) - 1)) == 0) {
#pragma unroll
            for (int w = 0; w < CNT; ++w) {
              const int n = (fr >> sh) * CNT + w;
              const int row = wm + 32 * (n >> 4) + 8 * ((n & 15) >> 2) + 4 * fg + (n & 3);
              s_dal[(wid % WN) * BM + row] = dal[w];
            }
          }
          lds_barrier();
          if (tid < t.rows) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) sum += s_dal[w * BM + tid];
            p.dalpha_part[int64_t(s_ment[tid]) * nt_count + t.n0 / BN] = sum;
          }
        }
      }
      return;
    }
    // Row-major outputs: each group of four rows of a column (the lane's
    // registers 4 vq .. 4 vq + 3) is transposed inside the lane quad, so a lane
    // stores four consecutive columns of one row in a single 8-byte (bf16) or
    // 16-byte (fp32) store.  Row scales (alpha) apply before the transpose.
    if constexpr (!QT) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ro = 32 * i + 8 * (v >> 2) + (v & 3);
          if (ro >= rows_left) continue;
          T* out = static_cast<T*>(p.out) + (t.row0 + rl + ro) * p.Nout + t.n0 + cl;
#pragma unroll
          for (int j = 0; j < TN; ++j)
            if (32 * j < cols_left) {
              if constexpr (KIND == KIND_GATEUP)
                out[32 * j] = from_f32<T>(silu_mul(acc[0][i][j][v], acc[NP - 1][i][j][v]));
            }
        }
      }
      return;
    }
    const int q4 = fr & 3;
    const int cq = t.n0 + (cl & ~3);  // first column of the lane's quad
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int ro0 = 32 * i + 8 * vq;
        const int ro = ro0 + q4;  // the lane's row after the transpose
        const bool row_ok = ro < rows_left;
        float a4[4] = {1.f, 1.f, 1.f, 1.f};
        int64_t ent = 0;
        if constexpr (META) {
#pragma unroll
          for (int w = 0; w < 4; ++w) a4[w] = s_malpha[rl + ro0 + w];
          ent = s_ment[rl + ro];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const bool ok = row_ok && 32 * j < cols_left;  // columns: the same for the quad
          const int col = cq + 32 * j;
          if constexpr (KGROUP) {
            const int64_t o = (int64_t(t.e) * p.M + t.row0 + rl + ro) * p.Nout + col;
#pragma unroll
            for (int q = 0; q < NP; ++q) {
              float b[4];
#pragma unroll
              for (int w = 0; w < 4; ++w) b[w] = acc[q][i][j][4 * vq + w];
              quad_transpose(b, q4);
              if (ok) store4<T>(static_cast<T*>(q == 0 ? p.out : p.out1) + o, b);
            }
          } else if constexpr (KIND == KIND_GATEUP) {
            float b[4];
#pragma unroll
            for (int w = 0; w < 4; ++w)
              b[w] = silu_mul(acc[0][i][j][4 * vq + w], acc[NP - 1][i][j][4 * vq + w]);
            quad_transpose(b, q4);
            if (ok) store4<T>(static_cast<T*>(p.out) + (t.row0 + rl + ro) * p.Nout + col, b);
          } else {
            // (with a K split: the chunk's raw sums, in grouped row order)
            float b[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) b[w] = acc[0][i][j][4 * vq + w] * (SPLIT ? 1.f : a4[w]);
            quad_transpose(b, q4);
            if constexpr (SPLIT) {
              const int64_t o = (int64_t(t.chunk) * p.M + t.row0 + rl + ro) * p.Nout + col;
              if (ok) store4<float>(p.partial + o, b);
            } else if constexpr (KIND == KIND_DOWN_Y) {
              const int64_t o = (ent / p.k) * p.Nout + col;
              if (ok) {
                if (p.residual != nullptr) {
                  float r[4];
                  load4<T>(static_cast<const T*>(p.residual) + o, r);
#pragma unroll
                  for (int w = 0; w < 4; ++w) b[w] = r[w] + b[w];
                }
                store4<T>(static_cast<T*>(p.out) + o, b);
              }
            } else {
              if (ok) store4<T>(static_cast<T*>(p.out) + ent * p.Nout + col, b);
            }
          }
        }
      }
    }
  };

  // ---- the block's tiles.  When S divides the number of K slices every tile
  // starts in slot 0 and the ring streams straight on into the next tile
  // (its first S slices are issued during this tile's last S steps);
  // otherwise each tile fills and drains the ring on its own.
  const bool stream = !KGROUP && !SPLIT && (KTu % S) == 0;
  Tile cur = decode(0);
  load_rows(cur, rid);
  make_src(cur, rid);
  Tile nxt = cur;
  if (stream && n_my > 1) {
    nxt = decode(1);
    load_rows(nxt, rid);
  }

  for (int cj = 0; cj < n_my; ++cj) {
    const bool has_next = cj + 1 < n_my;
    const bool xnext = stream && has_next;
    const int KT = cur.kt;
    zero_acc();
    if (cj == 0 || !stream) {
      // A tile that fills the ring on its own waits here for its first slice
      // anyway: its epilogue metadata and (dh) (g, u) pairs are fetched under
      // that wait instead of stalling one of its last K steps.
      if (!stream) {
        load_meta(cur);
        load_gu(cur);
      }
      // fill the ring with the tile's first slices, wait for slice 0
      const int npro = KT < S ? KT : S;
      for (int sl = 0; sl < npro; ++sl) issue(sl, slot_ptr(sl));
      if (npro == S) wait_vmcnt<(S - 1) * LPW>();
      else wait_vmcnt<0>();
      ring_barrier();
      frag_load(ring0, 0, fa0, fb0);
    }
    int kt = 0;
    // Groups of S steps with static slots (slice kt lives in slot kt % S).
    // In a group every step refills its slot with slice kt + S: of this tile,
    // or, in the last group of a streaming tile, of the next tile.
    for (; stream ? (kt < KT) : (kt + 2 * S - 1 < KT); kt += S) {
      const bool last_group = kt + S >= KT;
      if (last_group) {
        // this tile's slices are all issued: the sources move on to the next tile
        if (xnext) make_src(nxt, rid);
        load_meta(cur);
        load_gu(cur);
      }
      // the very last slices of the block: nothing left to fetch, drain
      const bool tail = last_group && !xnext;
      const bool refill = !last_group || xnext;
      const int ik = last_group ? kt + S - KT : kt + S;  // slice index (in its tile) to issue
      step(ring0, ring1, false, refill, ik);
      if constexpr (S == 2) {
        step(ring1, ring0, tail, refill, ik + 1);
      } else if constexpr (S == 3) {
        step(ring1, ring2, tail, refill, ik + 1);
        step(ring2, ring0, tail, refill, ik + 2);
      } else {
        step(ring1, ring2, tail, refill, ik + 1);
        step(ring2, ring3, tail, refill, ik + 2);
        step(ring3, ring0, tail, refill, ik + 3);
      }
    }
    // Non-streaming tiles: the remaining steps (fewer than 2S) with run-time
    // slots; in the last S - 1 of them there is nothing left to fetch.
    if (!stream) {
      for (; kt < KT; ++kt) {
        const int sl = kt % S;
        const bool more = kt + S < KT;
        step(slot_ptr(sl), slot_ptr(sl + 1 == S ? 0 : sl + 1), !more, more, kt + S);
      }
    }
    epilogue(cur);
    if (xnext) {
      cur = nxt;
      if (cj + 2 < n_my) {
        nxt = decode(cj + 2);
        load_rows(nxt, rid);
      }
    } else if (has_next) {
      cur = decode(cj + 1);
      load_rows(cur, rid);
      make_src(cur, rid);
    }
  }
}

// Blocks of one kernel that fit on the device at once (CUs x resident
// blocks per CU), queried once per kernel and device (`cached` belongs to the
// kernel: every instantiation of the launcher below has its own).
template <typename K>
int resident_blocks(K kernel, int threads, int (&cached)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

template <typename T, int BM, int BN, int WM, int WN, int RB, int S, int KIND>
hipError_t launch_gemm_t(const GemmParams& p, int64_t mtiles, const Launch& s) {
  const int64_t nt = (p.Nout + BN - 1) / BN;
  auto kernel = gemm_kernel<T, BM, BN, WM, WN, RB, S, KIND>;
  if constexpr (KindTraits<KIND>::KGROUP) {
    // one block per tile: eight per-XCD shares of every group's tiles
    const int64_t te = ((p.M + BM - 1) / BM) * nt;
    const int64_t groups = p.offsets != nullptr ? p.E : 1;
    const int64_t grid = 8 * groups * ((te + 7) / 8);
    if (te <= 0 || grid > 0x7fffffff) return te <= 0 ? hipSuccess : hipErrorInvalidValue;
    return launch_kernel(kernel, dim3(unsigned(grid)), dim3(64 * WM * WN), 0, s, p);
  } else {
    // work items: tiles (times the K chunks of a split down projection)
    const int64_t items = mtiles * nt * (KIND == KIND_DOWN_PARTIAL ? int64_t(p.ksplit) : 1);
    if (items <= 0) return hipSuccess;
    // persistent grid: at most the blocks resident at once, in whole rounds of
    // the 8 XCDs (blocks beyond the real item count exit at once)
    static int cached[64] = {};
    const int64_t cap = resident_blocks(kernel, 64 * WM * WN, cached) / 8 * 8;
    int64_t grid = (items + 7) / 8 * 8;
    if (grid > cap && cap >= 8) grid = cap;
    // in-block routing: one more block, which writes the routing outputs
    if (p.inl_topk != nullptr && p.inl_outputs != 0) ++grid;
    // router blocks riding on a decode gate/up launch
    if (KIND == KIND_GATEUP && p.rt_blocks > 0) grid += p.rt_blocks;
    return launch_kernel(kernel, dim3(unsigned(grid)), dim3(64 * WM * WN), 0, s, p);
  }
}

// Launches a shape only when it is valid for the kind (LDS ring within 156 KB,
// leaving room for the epilogue's tables; slice rows split evenly over the
// wavefronts; padded-group kinds need BM a multiple of 64).  A plain
// specialisation rather than if-constexpr, so every kernel that can be
// launched is instantiated at namespace scope with its host stub.
template <int BM, int BN, int WM, int WN, int RB, int S, int KIND>
constexpr bool shape_ok() {
  constexpr int R = KindTraits<KIND>::NA * BM + KindTraits<KIND>::NB * BN;
  constexpr int NW = WM * WN;
  constexpr int RPI = 1024 / RB;
  constexpr bool pad = KindTraits<KIND>::KGROUP || KIND == KIND_BWD_GU || KIND == KIND_BWD_DH;
  return S * R * RB <= 156 * 1024 && (R / RPI) % NW == 0 && BM % RPI == 0 && BN % RPI == 0 &&
         (S - 1) * (R / RPI / NW) < 64 && (BM / WM) % 32 == 0 && (BN / WN) % 32 == 0 &&
         (!pad || BM % 64 == 0) && BM <= 64 * NW;
}

template <typename T, int BM, int BN, int WM, int WN, int RB, int S, int KIND,
          bool OK = shape_ok<BM, BN, WM, WN, RB, S, KIND>()>
struct ShapeLauncher {
  static hipError_t run(const GemmParams&, int64_t, const Launch&) { return hipErrorInvalidValue; }
};
template <typename T, int BM, int BN, int WM, int WN, int RB, int S, int KIND>
struct ShapeLauncher<T, BM, BN, WM, WN, RB, S, KIND, true> {
  static hipError_t run(const GemmParams& p, int64_t mtiles, const Launch& s) {
    return launch_gemm_t<T, BM, BN, WM, WN, RB, S, KIND>(p, mtiles, s);
  }
};

// The instantiated launch shapes: (BM, BN, WM, WN, RB, S) = block tile, wave
// grid, LDS row bytes (K slice of RB / sizeof(T) elements), ring depth.
// Forward projections:
#define TOPMOE_GEMM_SHAPES_BF16(X)                                                        \
  X(128, 64, 2, 2, 128, 2) X(128, 64, 2, 2, 128, 3) X(128, 64, 2, 2, 64, 4)               \
  X(128, 128, 2, 2, 128, 2) X(128, 128, 2, 2, 128, 3) X(128, 128, 2, 2, 64, 4)            \
  X(64, 64, 2, 2, 128, 3) X(64, 64, 2, 2, 128, 4)                                          \
  X(256, 128, 4, 2, 64, 4) X(256, 128, 4, 2, 64, 3) X(256, 256, 4, 2, 64, 4)              \
  X(128, 128, 2, 4, 64, 4) X(256, 128, 4, 2, 128, 2) X(128, 128, 2, 4, 128, 3)            \
  X(128, 128, 2, 4, 128, 4) X(256, 64, 4, 2, 128, 3) X(256, 128, 4, 2, 128, 3)            \
  X(64, 128, 2, 4, 128, 3) X(256, 256, 4, 2, 128, 2)
#define TOPMOE_GEMM_SHAPES_F32(X) X(128, 64, 2, 2, 128, 2) X(64, 64, 2, 2, 128, 3)
// The backward's recomputed gate/up projection and its dh projection (their
// LDS also holds one staged transposed output tile where it fits; the dh
// epilogue's (g, u) words and du values make 256-row tiles spill):
#define TOPMOE_BWDGU_SHAPES_BF16(X)                                                       \
  X(256, 128, 4, 2, 128, 2) X(128, 128, 2, 4, 128, 2) X(256, 64, 4, 2, 128, 2)
#define TOPMOE_BWDDH_SHAPES_BF16(X) X(128, 128, 2, 4, 128, 3) X(128, 128, 2, 4, 128, 2)
#define TOPMOE_BWD_SHAPES_F32(X) X(128, 64, 2, 2, 128, 2) X(64, 64, 2, 2, 128, 3)
// Weight gradients:
#define TOPMOE_WGRAD_SHAPES_BF16(X)                                                       \
  X(128, 256, 2, 4, 128, 2) X(128, 128, 2, 4, 128, 3) X(256, 128, 4, 2, 128, 3)           \
  X(128, 128, 2, 2, 128, 3) X(64, 64, 2, 2, 128, 3)
#define TOPMOE_WGRAD_SHAPES_F32(X) X(128, 64, 2, 2, 128, 2) X(64, 64, 2, 2, 128, 3)

template <typename T, int KIND>
hipError_t launch_gemm_tiles(GemmShape sh, const GemmParams& p, int64_t mtiles, const Launch& s) {
#define TOPMOE_TRY_SHAPE(BM_, BN_, WM_, WN_, RB_, S_)                                     \
  if (sh.bm == (BM_) && sh.bn == (BN_) && sh.wm == (WM_) && sh.wn == (WN_) &&            \
      sh.rb == (RB_) && sh.stages == (S_))                                               \
    return ShapeLauncher<T, BM_, BN_, WM_, WN_, RB_, S_, KIND>::run(p, mtiles, s);
  if constexpr (KIND == KIND_BWD_GU) {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_BWDGU_SHAPES_BF16(TOPMOE_TRY_SHAPE)
    } else {
      TOPMOE_BWD_SHAPES_F32(TOPMOE_TRY_SHAPE)
    }
  } else if constexpr (KIND == KIND_BWD_DH) {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_BWDDH_SHAPES_BF16(TOPMOE_TRY_SHAPE)
    } else {
      TOPMOE_BWD_SHAPES_F32(TOPMOE_TRY_SHAPE)
    }
  } else if constexpr (KindTraits<KIND>::KGROUP) {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_WGRAD_SHAPES_BF16(TOPMOE_TRY_SHAPE)
    } else {
      TOPMOE_WGRAD_SHAPES_F32(TOPMOE_TRY_SHAPE)
    }
  } else {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_GEMM_SHAPES_BF16(TOPMOE_TRY_SHAPE)
    } else {
      TOPMOE_GEMM_SHAPES_F32(TOPMOE_TRY_SHAPE)
    }
  }
#undef TOPMOE_TRY_SHAPE
  return hipErrorInvalidValue;
}

// Whether launch_gemm_tiles<T, KIND> has shape `sh` (instantiated and valid).
template <typename T, int KIND>
bool shape_listed(const GemmShape& sh) {
#define TOPMOE_HAS_SHAPE(BM_, BN_, WM_, WN_, RB_, S_)                                     \
  if (sh.bm == (BM_) && sh.bn == (BN_) && sh.wm == (WM_) && sh.wn == (WN_) &&            \
      sh.rb == (RB_) && sh.stages == (S_))                                               \
    return shape_ok<BM_, BN_, WM_, WN_, RB_, S_, KIND>();
  if constexpr (KIND == KIND_BWD_GU) {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_BWDGU_SHAPES_BF16(TOPMOE_HAS_SHAPE)
    } else {
      TOPMOE_BWD_SHAPES_F32(TOPMOE_HAS_SHAPE)
    }
  } else if constexpr (KIND == KIND_BWD_DH) {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_BWDDH_SHAPES_BF16(TOPMOE_HAS_SHAPE)
    } else {
      TOPMOE_BWD_SHAPES_F32(TOPMOE_HAS_SHAPE)
    }
  } else if constexpr (KindTraits<KIND>::KGROUP) {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_WGRAD_SHAPES_BF16(TOPMOE_HAS_SHAPE)
    } else {
      TOPMOE_WGRAD_SHAPES_F32(TOPMOE_HAS_SHAPE)
    }
  } else {
    if constexpr (sizeof(T) == 2) {
      TOPMOE_GEMM_SHAPES_BF16(TOPMOE_HAS_SHAPE)
    } else {
      TOPMOE_GEMM_SHAPES_F32(TOPMOE_HAS_SHAPE)
    }
  }
#undef TOPMOE_HAS_SHAPE
  return false;
}

template <typename T>
bool shape_supported_dtype(int kind, const GemmShape& sh) {
  switch (kind) {
    case KIND_GATEUP: return shape_listed<T, KIND_GATEUP>(sh);
    case KIND_DOWN_Y: return shape_listed<T, KIND_DOWN_Y>(sh);
    case KIND_DOWN_SLOTS: return shape_listed<T, KIND_DOWN_SLOTS>(sh);
    case KIND_DOWN_PARTIAL: return shape_listed<T, KIND_DOWN_PARTIAL>(sh);
    case KIND_BWD_GU: return shape_listed<T, KIND_BWD_GU>(sh);
    case KIND_BWD_DH: return shape_listed<T, KIND_BWD_DH>(sh);
    case KIND_WGRAD2: return shape_listed<T, KIND_WGRAD2>(sh);
    case KIND_WGRAD1: return shape_listed<T, KIND_WGRAD1>(sh);
  }
  return false;
}

template <typename T>
hipError_t launch_gemm_dtype(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                             const Launch& s) {
  switch (kind) {
    case KIND_GATEUP: return launch_gemm_tiles<T, KIND_GATEUP>(sh, p, mtiles, s);
    case KIND_DOWN_Y: return launch_gemm_tiles<T, KIND_DOWN_Y>(sh, p, mtiles, s);
    case KIND_DOWN_SLOTS: return launch_gemm_tiles<T, KIND_DOWN_SLOTS>(sh, p, mtiles, s);
    case KIND_DOWN_PARTIAL: return launch_gemm_tiles<T, KIND_DOWN_PARTIAL>(sh, p, mtiles, s);
    case KIND_BWD_GU: return launch_gemm_tiles<T, KIND_BWD_GU>(sh, p, mtiles, s);
    case KIND_BWD_DH: return launch_gemm_tiles<T, KIND_BWD_DH>(sh, p, mtiles, s);
    case KIND_WGRAD2: return launch_gemm_tiles<T, KIND_WGRAD2>(sh, p, mtiles, s);
    case KIND_WGRAD1: return launch_gemm_tiles<T, KIND_WGRAD1>(sh, p, mtiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace topmoe
