// HIP kernels of the Julia-1 forward pass for gfx950 (CDNA4, 64-wide waves).
//
// GEMMs and attention run on matrix cores: v_mfma_f32_16x16x32_bf16 in the
// bf16 mode, v_mfma_f32_16x16x4_f32 in the FP32 mode, FP32 accumulation in
// both.  Every operand fragment holds 8 consecutive K elements per lane (lane
// group g = lane / 16 owns k = 8g .. 8g+7 of a 32-wide K step); the FP32 mode
// feeds the same fragment to eight 16x16x4 steps, so one tiling serves both.
// Row-wise work (LayerNorm, softmax over options, dot products) uses
// wavefront reductions.
#include <type_traits>

#include "jl_device.h"

// No FMA contraction: unrolled code handles each row of a tile in its own
// instruction sequence, and a contraction the compiler applies to some of
// those sequences and not to others would make a row's rounding depend on
// its place in the tile, and so on how the batch was packed.
#pragma clang fp contract(off)

namespace jl {
namespace {
using namespace dev;

// ---------------------------------------------------------------------------
// embedding gather + LayerNorm (gain only); positions and sequence ids
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ ids,
                                                    const float *__restrict__ emb,
                                                    const float *__restrict__ gain, int T,
                                                    const int *__restrict__ seq_offsets, int n_seqs,
                                                    float *__restrict__ x, int *__restrict__ pos,
                                                    int *__restrict__ tok_seq) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int id = ids[t];
  const bool ok = id >= 0 && id < kVocab;
  const float *e = emb + (size_t)(ok ? id : 0) * kWidth;
  float v[6], s = 0.f;
#pragma unroll
  for (int i = 0; i < 6; ++i) { v[i] = e[lane + 64 * i]; s += v[i]; }
  const float mean = wave_sum(s) * (1.0f / kWidth);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 6; ++i) { const float d = v[i] - mean; q += d * d; }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / kWidth) + kLnEps);
  float *xr = x + (size_t)t * kWidth;
#pragma unroll
  for (int i = 0; i < 6; ++i) xr[lane + 64 * i] = ok ? (v[i] - mean) * rstd * gain[lane + 64 * i] : NAN;
  if (lane == 0) {
    int lo = 0, hi = n_seqs - 1;  // last b with seq_offsets[b] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_offsets[mid] <= t) lo = mid; else hi = mid - 1;
    }
    pos[t] = t - seq_offsets[lo];
    tok_seq[t] = lo;
  }
}

// ---------------------------------------------------------------------------
// GEMM: C = A . W^T (A [M, K] activations, W [N, K] weights, both K-contiguous).
//
// 256 threads as 2 x 2 waves; block tile BM x BN, wave tile (BM/2) x (BN/2),
// K staged in steps of BK (64 bf16 / 32 FP32 elements) through a double-
// buffered LDS tile.  LDS holds the tiles in matrix-core fragment order: one
// block of 64 lanes x 8 elements covers 16 rows x 32 k, lane (r + 16 c) holding
// row r, k = 8c .. 8c+7.  A wave stages one such block per global load (16
// rows x 64 contiguous bytes), writes it to LDS linearly and every fragment
// read is one linear 16-byte read per lane: no bank conflicts either way.
// LayerNorm, where the model has one, is applied beforehand by
// ln_rows_kernel, once per row, or, when the grid takes 64-row tiles, by the
// GEMM itself on its rows (the same arithmetic, so the same operands).
//
// The grid is 1-D.  Work-groups are dispatched to the 8 XCDs round-robin, so
// block b is remapped to tile t such that every XCD owns a contiguous run of
// tiles: all N-tiles of an M-block then share one XCD's L2.
// ---------------------------------------------------------------------------

// The shift of a LayerNorm that has none, for the GEMM's fused LayerNorm:
// adding + 0 from memory keeps the loads and the arithmetic free of branches
// and selects (and equals the LayerNorm kernel's + 0).
__device__ float g_ln_zero_shift[kWidth];

template <typename T> struct GemmBK;
template <> struct GemmBK<bf16> { static constexpr int v = 64; };
template <> struct GemmBK<float> { static constexpr int v = 32; };

// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations (vmcnt in bits 3:0 and 15:14) and leaves the other counters free.
constexpr int vm_wait_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// 16 bytes per lane from rows at `base` (lane byte offset voff, scalar byte
// offset soff) straight into LDS: lane i lands at dst + 16 i.  A device
// function of its own: the GEMM's lambdas are also compiled for the host,
// which has no buffer resources.
typedef __attribute__((address_space(3))) void lds_void;
__device__ inline void buffer_load_lds16(const void *base, lds_void *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000), dst, 16, voff,
      soff, 0, 0);
}

__device__ inline int xcd_tile(int b, int n_tiles) {
  const int per = n_tiles >> 3, rem = n_tiles & 7, x = b & 7, local = b >> 3;
  return x * per + min(x, rem) + local;
}

template <typename T, int BM, int BN, int EM, int NSTAGE, bool LNA = false, int KFIX = 0, bool RF = false,
          bool F8 = false>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, int tiles_n, int n_tiles) {
  constexpr int BK = GemmBK<T>::v, KS = BK / 32;           // 32-wide k sub-steps per stage
  constexpr int TM = BM / 2, TN = BN / 2;                   // wave tile
  constexpr int MT = TM / 16, NT = TN / 16;
  constexpr int FE = 8;                                      // elements per lane per fragment
  constexpr int BLK = 64 * FE;                               // elements per fragment block
  constexpr int A_BLKS = (BM / 16) * KS, B_BLKS = (BN / 16) * KS;
  constexpr int A_PER_WAVE = A_BLKS / 4, B_PER_WAVE = B_BLKS / 4;
  static_assert(A_BLKS % 4 == 0 && B_BLKS % 4 == 0, "tile must split over 4 waves");
  static_assert(NT % 4 == 0 || EM == E_RESID || EM == E_RELU,
                "GEGLU and RoPE epilogues pair columns within 64-column groups");
  // bf16: an NSTAGE-stage pipeline whose loads go straight from memory into
  // LDS (16 bytes per lane, lane i at block offset 16 i: the fragment order),
  // without staging registers.  The first NSTAGE K-steps are issued up front
  // and step kt refills the buffer step kt - 1 read, so NSTAGE - 1 steps stay
  // in flight; with NSTAGE >= K / BK (6 stages for K = 384, for grids that fit
  // the CUs in one or two rounds) the whole K arrives in one memory round
  // trip.  2 stages for larger grids leave LDS for more resident work-groups.
  // FP32: two LDS stages filled through registers, NSTAGE - 1 K-steps in
  // flight (register slot kt % (NSTAGE - 1)); one-round grids take 4, so that
  // a K = 384 product pays 3 memory round trips instead of 12.
  // Each bf16 stage buffer is a variable of its own and the K loop is
  // unrolled over the stages: the compiler then knows which buffer each
  // in-flight LDS load writes and adds no wait of its own before reading
  // another.  With K fixed at compile time (KFIX; the fused LayerNorm's
  // K = 384) the K loop unrolls completely and every wait is exact; with a
  // run-time K the compiler drains all loads once per round of stages.
  //
  // LNA (bf16, BM = 64, K = 384): A = LayerNorm(g.ln_x) rows, normalized by
  // the work-group itself into an LDS tile that holds all of K; only W
  // streams through the stages.  The rows and the LayerNorm parameters are
  // loaded first and normalized while the weight stages stream in (RF); an
  // identity pre-norm (no gain) issues the stages first, then the rows, and
  // once the rows are in every stage has landed.
  constexpr bool kDma = std::is_same<T, bf16>::value;
  constexpr int NS = kDma ? NSTAGE : 2;
  static_assert(NS >= 2 && NS <= 6, "stages");
  static_assert(!LNA || (kDma && BM == 64), "fused LayerNorm: bf16, 64-row tiles");
  // F8: e4m3 operands.  The LayerNorm rows are scaled per row (largest
  // magnitude -> 448) and converted into an LDS tile of e4m3 codes; W holds
  // e4m3 codes with a scale per row (w_scale).  Both tiles keep a 16-row
  // group's codes in 16-byte chunks: byte k % 16 of chunk (k / 16) * 16 + row,
  // so that a lane's 8 codes of a 32-k step are one 8-byte read, and a weight
  // stage (64 k of 16 rows, 1 KB) is one 16-byte LDS-direct load per lane.
  // The products accumulate in FP32 and the epilogue multiplies by both scales.
  static_assert(!F8 || (LNA && RF && (EM == E_STORE || EM == E_GEGLU)), "e4m3: LayerNorm with a gain, QKV or GEGLU");
  constexpr int SBE = kDma ? (F8 ? B_BLKS * BLK / 2 : B_BLKS * BLK) : 1;  // stage elements of W
  constexpr int KA = kWidth / 32;  // k sub-steps of the resident A tile
  constexpr int SA = kDma && !LNA ? A_BLKS * BLK : 1;
  __shared__ __attribute__((aligned(16))) T sA[kDma ? 1 : NS][A_BLKS * BLK];  // FP32 stages
  __shared__ __attribute__((aligned(16))) T sB[kDma ? 1 : NS][B_BLKS * BLK];
  __shared__ __attribute__((aligned(16))) T sAk[LNA && !F8 ? BM * kWidth : 1];
  __shared__ __attribute__((aligned(16))) uint8_t sA8[F8 ? BM * kWidth : 1];
  __shared__ float sSa[F8 ? BM : 1];  // e4m3 row scales
  __shared__ __attribute__((aligned(16))) T sA0[SA], sB0[SBE];
  __shared__ __attribute__((aligned(16))) T sA1[SA], sB1[SBE];
  __shared__ __attribute__((aligned(16))) T sA2[NS > 2 ? SA : 1], sB2[NS > 2 ? SBE : 1];
  __shared__ __attribute__((aligned(16))) T sA3[NS > 3 ? SA : 1], sB3[NS > 3 ? SBE : 1];
  __shared__ __attribute__((aligned(16))) T sA4[NS > 4 ? SA : 1], sB4[NS > 4 ? SBE : 1];
  __shared__ __attribute__((aligned(16))) T sA5[NS > 5 ? SA : 1], sB5[NS > 5 ? SBE : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t = xcd_tile(g.rev ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x, n_tiles);
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  const int M = g.M;
  const int lr = lane & 15, lc = (lane >> 4) * 8;           // lane's row / k offset inside a block

  // fragment block q of a tile: row group q / KS, k sub-step q % KS
  const T *Ab = (const T *)g.A, *Wb = (const T *)g.W;
  constexpr int PD = kDma ? 1 : NSTAGE - 1;  // FP32: K-steps in flight through registers
  Frag<T> ra[PD][A_PER_WAVE], rb[PD][B_PER_WAVE];
  // K-step kt (clamped to the last: a load past the end is never stored) into register slot r
  auto load_stage = [&](int kt, int r) {
    const int k0 = min(kt, (KFIX ? KFIX : g.K) / BK - 1) * BK + lc;
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) {
      const int q = wave * A_PER_WAVE + i;
      const int row = min(m0 + (q / KS) * 16 + lr, M - 1);
      ra[r][i] = load_frag(Ab + (size_t)row * g.lda + k0 + (q % KS) * 32);
    }
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int q = wave * B_PER_WAVE + i;
      rb[r][i] = load_frag(Wb + (size_t)(n0 + (q / KS) * 16 + lr) * g.ldw + k0 + (q % KS) * 32);
    }
  };
  auto store_stage = [&](int buf, int r) {
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i) store_frag(&sA[buf][(wave * A_PER_WAVE + i) * BLK + lane * FE], ra[r][i]);
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) store_frag(&sB[buf][(wave * B_PER_WAVE + i) * BLK + lane * FE], rb[r][i]);
  };

  f32x4 acc[MT][NT];  // zeroed just before the K loop: no registers held through the prologue
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  constexpr int KC = LNA ? kWidth : KFIX;  // K when fixed at compile time
  // RF (a fused LayerNorm with a gain): the rows are loaded first and
  // normalized while the weight stages stream in.  Without RF (the identity
  // pre-norm of the first layer) every weight stage goes first and lands with
  // the rows (kAllIn below).
  constexpr bool kRowsFirst = LNA && RF;
  static_assert(!RF || LNA, "rows first: fused LayerNorm only");
  static_assert(KC % BK == 0, "K steps");
  const int KT = KC ? KC / BK : g.K / BK;
  constexpr bool kAllIn = LNA && !kRowsFirst && NSTAGE * BK >= kWidth;
  // rows first with every stage issued up front: the RoPE table rows, which
  // need the positions, are read right after the LayerNorm, and the stage
  // waits count them (younger than every stage)
  constexpr bool kRopeEarly = kRowsFirst && EM == E_STORE && NSTAGE * BK >= kWidth;
  // fused LayerNorm: each wave normalizes 16 rows, 4 at a time, one per
  // 16-lane row of the wave (lane j: columns 64 c + 4 j .. + 3, c = 0..5),
  // with all their loads in flight; the gain and shift columns of a lane are
  // the same in every pass.  The rows are loaded first: a wait the compiler
  // places after the later, branchy parameter loads then only waits for data
  // the LayerNorm needs next.
  constexpr int LP = LNA ? BM / 16 : 1;  // passes of 4 rows per wave
  const int lj = lane & 15;
  f32x4 lnx[LP][6], lng[6], lns[6];
  auto ln_load = [&]() {
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < LP; ++p) {
      const int row = min(m0 + wave * (BM / 4) + 4 * p + (lane >> 4), M - 1);
      const float *xr = g.ln_x + (size_t)row * kWidth + 4 * lj;
#pragma unroll
      for (int c = 0; c < 6; ++c) lnx[p][c] = *reinterpret_cast<const f32x4 *>(xr + 64 * c);
    }
    if constexpr (kRowsFirst) {
      // always normalized (the launcher checks the gain); an absent shift is
      // read as zeros: loads under no branch, so no merge copies and no
      // early waits
      const float *sh = g.ln_shift ? g.ln_shift : g_ln_zero_shift;
#pragma unroll
      for (int c = 0; c < 6; ++c) {
        lng[c] = *reinterpret_cast<const f32x4 *>(g.ln_gain + 64 * c + 4 * lj);
        lns[c] = *reinterpret_cast<const f32x4 *>(sh + 64 * c + 4 * lj);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 6; ++c) lng[c] = lns[c] = z;  // absent shift: + 0
      if (g.ln_gain != nullptr) {
#pragma unroll
        for (int c = 0; c < 6; ++c) lng[c] = *reinterpret_cast<const f32x4 *>(g.ln_gain + 64 * c + 4 * lj);
        if (g.ln_shift) {
#pragma unroll
          for (int c = 0; c < 6; ++c) lns[c] = *reinterpret_cast<const f32x4 *>(g.ln_shift + 64 * c + 4 * lj);
        }
      }
    }
  };
  auto ln_finish = [&]() {
    const bool norm = kRowsFirst || g.ln_gain != nullptr;
#pragma unroll
    for (int p = 0; p < LP; ++p) {
      const int rl = wave * (BM / 4) + 4 * p + (lane >> 4);
      f32x4 y[6];
#pragma unroll
      for (int c = 0; c < 6; ++c) y[c] = lnx[p][c];
      if (norm) {
        float mean, rstd;
        ln_row16(lnx[p], mean, rstd);
#pragma unroll
        for (int c = 0; c < 6; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) y[c][e] = (y[c][e] - mean) * rstd * lng[c][e] + lns[c][e];
      }
      if constexpr (F8) {
        float am = 0.f;
#pragma unroll
        for (int c = 0; c < 6; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) am = fmaxf(am, fabsf(y[c][e]));
        am = row16_max(am);
        // codes of y 448 / amax, the row's scale amax / 448
        const float rc = am > 0.f ? 448.0f / am : 1.0f, sc = am > 0.f ? am / 448.0f : 1.0f;
        const int r16 = rl & 15;
        uint8_t *grp = &sA8[(rl >> 4) * 16 * kWidth];
#pragma unroll
        for (int c = 0; c < 6; ++c) {
          const int k = 64 * c + 4 * lj;
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[c][0] * rc, y[c][1] * rc, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(y[c][2] * rc, y[c][3] * rc, w, true);
          const unsigned a3 =
              (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)&grp[16 * ((k >> 4) * 16 + r16) + (k & 15)];
          asm volatile("ds_write_b32 %0, %1" ::"v"(a3), "v"(w));
        }
        if (lj == 0) {
          const unsigned a3 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float *)&sSa[rl];
          asm volatile("ds_write_b32 %0, %1" ::"v"(a3), "v"(__float_as_uint(sc)));
        }
        continue;
      }
#pragma unroll
      for (int c = 0; c < 6; ++c) {
        // (row rl, k = 64 c + 4 lj): block (rl / 16, k / 32), lane (rl % 16) + 16 ((k % 32) / 8), element k % 8
        const int k = 64 * c + 4 * lj;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)y[c][e];
        T *dst = &sAk[((rl >> 4) * KA + (k >> 5)) * BLK + ((rl & 15) + 16 * ((k & 31) >> 3)) * FE + (k & 7)];
        if constexpr (kRowsFirst) {
          // the weight stages' LDS-direct loads are still in flight, into
          // other LDS buffers; a plain store would make the compiler wait
          // for all of them.  The lgkmcnt(0) before the first barrier of the
          // K loop completes these stores.
          typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
          const unsigned a3 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) T *)dst;
          asm volatile("ds_write_b64 %0, %1" ::"v"(a3), "v"(__builtin_bit_cast(u32x2, v)));
        } else {
          *reinterpret_cast<bf16x4 *>(dst) = v;
        }
      }
    }
  };
  // epilogue coordinates: acc[i][j][r] = C[row0 + 16i + r][col0 + 16j]
  const int row0 = m0 + wm * TM + (lane >> 4) * 4;
  const int wcol = n0 + wn * TN;            // first of this wave's TN columns
  const int col0 = wcol + lr;
  // Epilogue operands that do not depend on the product (bias, RoPE table
  // rows, the residual) are all read before the first store: a load that
  // follows a store to C may alias it, and the compiler would then wait for
  // every earlier memory operation at each row.  A tile of at most 64 rows
  // (kHoist) reads them before the K loop (the RoPE table rows, which need
  // the positions: right after a fused LayerNorm that has every weight stage
  // in flight, else before the epilogue), larger tiles one 16-row group at a
  // time.
  constexpr bool kHoist = kDma && BM <= 64;
  constexpr int HG = kHoist ? MT : 1;  // row groups held at once
  const bool has_bias = g.bias != nullptr;
  const bool rope = EM == E_STORE && g.rope_cos != nullptr;
  // the RoPE reads take no branch (a load under a branch makes the compiler
  // wait for it at the merge, before the weight stages are even issued):
  // without a table they read zeros at position 0
  const int *pos_p = rope ? g.pos : (const int *)g_ln_zero_shift;
  const int pos_step = rope ? 1 : 0;
  const float *cos_p = rope ? g.rope_cos : g_ln_zero_shift, *sin_p = rope ? g.rope_sin : g_ln_zero_shift;
  float bias_v[NT];
  float wsc_v[F8 ? NT : 1];  // e4m3 weight row scales of this lane's columns
  int rpos[HG][4];
  float rcs[HG][4][4];  // per row: cos and sin of d = lr, then of d = 16 + lr
  float res[EM == E_RESID ? HG : 1][4][EM == E_RESID ? NT : 1];
  // unconditional loads (without a bias they read the output row, and the
  // epilogue adds nothing): a load under a branch would need a copy at the
  // merge, and the copy an early wait
  auto load_bias = [&]() {
    const float *b = has_bias ? g.bias : (const float *)g.C;
#pragma unroll
    for (int j = 0; j < NT; ++j) bias_v[j] = b[col0 + j * 16];
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < NT; ++j) wsc_v[j] = g.w_scale[col0 + j * 16];
    }
  };
  auto load_pos = [&](int i, int h) {
#pragma unroll
    for (int r = 0; r < 4; ++r) rpos[h][r] = pos_p[min(row0 + i * 16 + r, M - 1) * pos_step];
  };
  auto load_rope = [&](int h) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = rpos[h][r] * 32 + j * 16 + lr;
        rcs[h][r][2 * j] = cos_p[q];
        rcs[h][r][2 * j + 1] = sin_p[q];
      }
  };
  auto load_res = [&](int i, int h) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float *C = (const float *)g.C + (size_t)min(row0 + i * 16 + r, M - 1) * g.ldc + col0;
#pragma unroll
      for (int j = 0; j < NT; ++j) res[h][r][j] = C[j * 16];
    }
  };
  // the operands a tile of at most 64 rows reads before its K loop
  auto load_hoisted = [&]() {
    load_bias();
    if constexpr (kHoist) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if constexpr (EM == E_RESID) load_res(i, i);
        if constexpr (EM == E_STORE) load_pos(i, i);
      }
    }
  };
  // A fragment (row sub-tile i of this wave, k sub-step ks of K-step kt)
  auto a_frag = [&](const T *cA, int kt, int i, int ks) -> Frag<T> {
    if constexpr (LNA) return load_frag(&sAk[((wm * MT + i) * KA + kt * KS + ks) * BLK + lane * FE]);
    else return load_frag(&cA[((wm * MT + i) * KS + ks) * BLK + lane * FE]);
  };
  // e4m3 products over 128 k (K-steps kt - 1 and kt, kt odd) on the
  // 16x16x128 fp8 matrix-core product (unit block scales): lane (row lr,
  // group g) supplies k = 32 g .. 32 g + 31 of the window, two 16-byte chunks
  // of each operand; W's first half comes from stage buffer cP, the second
  // from cB.  The product sums over k, so only the pairing of A and W codes
  // matters, not their order.
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  typedef int i32x4v __attribute__((ext_vector_type(4)));
  auto compute8 = [&](const T *cP, const T *cB, int kt) {
    const int g = lane >> 4;
    const uint8_t *B8 = (const uint8_t *)((g >> 1) ? cB : cP);
    const int ca = (kt - 1) * 4 + 2 * g;  // first A chunk of the lane
    const int cb = (g & 1) * 2;           // first W chunk inside the stage
    i32x8 fa[MT], fb[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const uint8_t *a = &sA8[(wm * MT + i) * 16 * kWidth + 16 * (ca * 16 + lr)];
      const i32x4v lo = *reinterpret_cast<const i32x4v *>(a), hi = *reinterpret_cast<const i32x4v *>(a + 256);
      fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint8_t *b = &B8[(wn * NT + j) * 1024 + 16 * (cb * 16 + lr)];
      const i32x4v lo = *reinterpret_cast<const i32x4v *>(b), hi = *reinterpret_cast<const i32x4v *>(b + 256);
      fb[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  };
  auto compute = [&](const T *cA, const T *cB, int kt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag<T> fa[MT], fb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = a_frag(cA, kt, i, ks);
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[j] = load_frag(&cB[((wn * NT + j) * KS + ks) * BLK + lane * FE]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) mfma(acc[i][j], fa[i], fb[j]);
    }
  };
  if constexpr (kDma) {
    constexpr int LPS = F8 ? BN / 64 : (LNA ? 0 : A_PER_WAVE) + B_PER_WAVE;  // loads per stage and wave
    auto bufA = [&](auto Bc) -> T * {
      constexpr int B = decltype(Bc)::value;
      if constexpr (B == 0) return sA0;
      else if constexpr (B == 1) return sA1;
      else if constexpr (B == 2) return sA2;
      else if constexpr (B == 3) return sA3;
      else if constexpr (B == 4) return sA4;
      else return sA5;
    };
    auto bufB = [&](auto Bc) -> T * {
      constexpr int B = decltype(Bc)::value;
      if constexpr (B == 0) return sB0;
      else if constexpr (B == 1) return sB1;
      else if constexpr (B == 2) return sB2;
      else if constexpr (B == 3) return sB3;
      else if constexpr (B == 4) return sB4;
      else return sB5;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    // stage kt -> LDS buffer pair (dA, dB), one 1 KB fragment block per load
    // Buffer loads into LDS: a lane's byte offset inside the tile's rows is
    // fixed for all K-steps (one VGPR per fragment block), the K-step's
    // offset is a scalar, so the stages need no per-load address registers
    // (reusing one while its load is in flight would make the compiler wait
    // for that load).  Offsets count from the tile's first row.
    int voA[LNA ? 1 : A_PER_WAVE], voB[B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < (LNA ? 0 : A_PER_WAVE); ++i) {
      const int q = wave * A_PER_WAVE + i;
      const int row = min(m0 + (q / KS) * 16 + lr, M - 1) - m0;
      voA[i] = (row * g.lda + lc + (q % KS) * 32) * (int)sizeof(T);
    }
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int q = wave * B_PER_WAVE + i;
      voB[i] = (((q / KS) * 16 + lr) * g.ldw + lc + (q % KS) * 32) * (int)sizeof(T);
    }
    const T *tileA = Ab + (size_t)(LNA ? 0 : m0) * g.lda, *tileB = Wb + (size_t)n0 * g.ldw;
    // F8: 16-row group q of the stage from lane (row lane % 16, k chunk lane / 16)
    int voB8[F8 ? BN / 64 : 1];
    const uint8_t *tileB8 = (const uint8_t *)g.W + (size_t)n0 * g.ldw;
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < BN / 64; ++i) voB8[i] = ((wave * (BN / 64) + i) * 16 + lr) * g.ldw + (lane >> 4) * 16;
    }
    auto issue_stage = [&](int kt, T *dA, T *dB) {
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < BN / 64; ++i)
          buffer_load_lds16(tileB8, (lds_void *)((uint8_t *)dB + (wave * (BN / 64) + i) * 1024), voB8[i], kt * 64);
        return;
      }
      const int so = kt * BK * (int)sizeof(T);
#pragma unroll
      for (int i = 0; i < (LNA ? 0 : A_PER_WAVE); ++i) {
        const int q = wave * A_PER_WAVE + i;
        buffer_load_lds16(tileA, (lds_void *)&dA[q * BLK], voA[i], so);
      }
#pragma unroll
      for (int i = 0; i < B_PER_WAVE; ++i) {
        const int q = wave * B_PER_WAVE + i;
        buffer_load_lds16(tileB, (lds_void *)&dB[q * BLK], voB[i], so);
      }
    };
    // wait until at most `later` stages younger than the current one are in
    // flight, besides the R loads issued after the last stage (the
    // immediate must be a constant)
    auto wait_n = [&](auto Rc, int later) {
      constexpr int R = decltype(Rc)::value;
      switch (later) {
        case 0: __builtin_amdgcn_s_waitcnt(vm_wait_imm(R)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vm_wait_imm(LPS + R)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * LPS + R)); break;
        case 3: __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * LPS + R)); break;
        case 4: __builtin_amdgcn_s_waitcnt(vm_wait_imm(4 * LPS + R)); break;
        default: __builtin_amdgcn_s_waitcnt(vm_wait_imm(5 * LPS + R)); break;
      }
    };
    constexpr int kRopeLoads = MT * 16;  // table reads per lane: 4 rows x 2 halves x (cos, sin)
    auto wait_stages = [&](int later) { wait_n(std::integral_constant<int, kRopeEarly ? kRopeLoads : 0>(), later); };
    // K-step kt from buffer B (= kt % NS): wait for this wave's loads of the
    // step, then a bare barrier: every wave's loads of the step have landed
    // and every wave is done reading the previous step's buffer, which step
    // kt (> 0) refills.  Younger stages in flight at the wait: the other
    // up-front stages (kt = 0), else those issued by steps 1 .. kt - 1.
    // With every stage in before the LayerNorm (kAllIn), one barrier after
    // the A tile's LDS stores is all the loop needs.
    auto step = [&](int kt, auto Bc) {
      constexpr int B = decltype(Bc)::value;
      if constexpr (kAllIn) {
        if (kt == 0) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the A tile's LDS stores
          __builtin_amdgcn_s_barrier();
        }
      } else {
        wait_stages(kt == 0 ? min(KT, NS) - 1 : min(KT - 1 - kt, NS - 2));
        if constexpr (LNA)
          if (kt == 0) __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the A tile's LDS stores
        __builtin_amdgcn_s_barrier();
        using Next = std::integral_constant<int, (B + NS - 1) % NS>;
        if (kt > 0 && kt + NS - 1 < KT) issue_stage(kt + NS - 1, bufA(Next()), bufB(Next()));
      }
      if constexpr (F8) {
        using Prev = std::integral_constant<int, (B + NS - 1) % NS>;
        if (kt & 1) compute8(bufB(Prev()), bufB(Bc), kt);
      } else {
        compute(bufA(Bc), bufB(Bc), kt);
      }
    };
    // loads older than every stage never hold up a stage wait (the
    // scheduling barrier keeps the scheduler from sinking them towards their
    // use, behind the stages)
    if constexpr (kRowsFirst) {
      ln_load();
      load_hoisted();
    } else if constexpr (!LNA) {
      load_hoisted();
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_stage(0, sA0, sB0);
    if (KT > 1) issue_stage(1, sA1, sB1);
    if constexpr (NS > 2)
      if (KT > 2) issue_stage(2, bufA(I2()), bufB(I2()));
    if constexpr (NS > 3)
      if (KT > 3) issue_stage(3, bufA(I3()), bufB(I3()));
    if constexpr (NS > 4)
      if (KT > 4) issue_stage(4, bufA(I4()), bufB(I4()));
    if constexpr (NS > 5)
      if (KT > 5) issue_stage(5, bufA(I5()), bufB(I5()));
    if constexpr (LNA) {
      if constexpr (!kRowsFirst) {
        ln_load();
        load_hoisted();
      }
      // keep the stage loads ahead of the LayerNorm arithmetic: the scheduler
      // would otherwise sink them below it, and the weights would only be
      // requested once the LayerNorm is done
      __builtin_amdgcn_sched_barrier(0);
      ln_finish();  // weights first: waits for the rows, younger than every stage
      if constexpr (EM == E_STORE && (kAllIn || kRopeEarly)) {
        // rows first: counted by the stage waits (every stage was issued
        // before); weights first: every stage has landed
#pragma unroll
        for (int i = 0; i < MT; ++i) load_rope(i);
      }
    }
    zero_acc();
    auto round = [&](int kt) {  // steps kt .. kt + NS - 1
      step(kt, I0());
      if (kt + 1 < KT) step(kt + 1, I1());
      if constexpr (NS > 2)
        if (kt + 2 < KT) step(kt + 2, I2());
      if constexpr (NS > 3)
        if (kt + 3 < KT) step(kt + 3, I3());
      if constexpr (NS > 4)
        if (kt + 4 < KT) step(kt + 4, I4());
      if constexpr (NS > 5)
        if (kt + 5 < KT) step(kt + 5, I5());
    };
    if constexpr (KC != 0) {
#pragma unroll
      for (int kt = 0; kt < KT; kt += NS) round(kt);
    } else {
      for (int kt = 0; kt < KT; kt += NS) round(kt);
    }
  } else {
    zero_acc();
    load_bias();
#pragma unroll
    for (int r = 0; r < PD; ++r) load_stage(r, r);
    store_stage(0, 0);
    __syncthreads();
    // step kt, slot r = kt % PD: the slot's K-step reached LDS at the end of
    // step kt - 1 (or before the loop), so it takes K-step kt + PD
    auto fstep = [&](int kt, auto Rc) {
      constexpr int r = decltype(Rc)::value;
      load_stage(kt + PD, r);
      compute(sA[kt & 1], sB[kt & 1], kt);
      if (kt + 1 < KT) store_stage((kt + 1) & 1, (r + 1) % PD);
      __syncthreads();
    };
    auto fround = [&](int kt0) {
      fstep(kt0, std::integral_constant<int, 0>());
      if constexpr (PD > 1)
        if (kt0 + 1 < KT) fstep(kt0 + 1, std::integral_constant<int, (PD > 1 ? 1 : 0)>());
      if constexpr (PD > 2)
        if (kt0 + 2 < KT) fstep(kt0 + 2, std::integral_constant<int, (PD > 2 ? 2 : 0)>());
      if constexpr (PD > 3)
        if (kt0 + 3 < KT) fstep(kt0 + 3, std::integral_constant<int, (PD > 3 ? 3 : 0)>());
    };
    // with K fixed at compile time the loop unrolls completely: no slot value
    // crosses a loop back edge, where the register copies would wait for loads
    if constexpr (KC != 0) {
#pragma unroll
      for (int kt0 = 0; kt0 < KT; kt0 += PD) fround(kt0);
    } else {
      for (int kt0 = 0; kt0 < KT; kt0 += PD) fround(kt0);
    }
  }

  // epilogue, one 16-row group at a time
  if constexpr (EM == E_STORE && kHoist && !kAllIn && !kRopeEarly) {
#pragma unroll
    for (int i = 0; i < MT; ++i) load_rope(i);
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int h = kHoist ? i : 0;
    if constexpr (!kHoist) {
      if constexpr (EM == E_RESID) load_res(i, 0);
      if constexpr (EM == E_STORE) {
        load_pos(i, 0);
        load_rope(0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + i * 16 + r;
      if (row >= M) continue;
      float v[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) v[j] = acc[i][j][r];
      if constexpr (F8) {
        const float sa = sSa[row - m0];
#pragma unroll
        for (int j = 0; j < NT; ++j) v[j] *= sa * wsc_v[j];
      }
      if (EM == E_GEGLU) {  // sub-tiles (2p, 2p+1) hold matching GELU and gate columns
        T *C = (T *)g.C + (size_t)row * g.ldc + wcol / 2 + lr;
#pragma unroll
        for (int p = 0; p < NT / 2; ++p) {  // bf16 output: the cheaper erf is exact enough
          const float ge = std::is_same<T, bf16>::value ? gelu_erf_fast(v[2 * p]) : gelu_erf(v[2 * p]);
          C[p * 16] = to_elem<T>(ge * v[2 * p + 1]);
        }
        continue;
      }
      if (has_bias) {
#pragma unroll
        for (int j = 0; j < NT; ++j) v[j] += bias_v[j];
      }
      if (EM == E_STORE) {
        if (rope) {  // each 64-column group is one head: pairs (d, d + 32)
#pragma unroll
          for (int hb = 0; hb < NT / 4; ++hb) {
            if (wcol + hb * 64 >= g.rope_cols) break;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float c = rcs[h][r][2 * j], sn = rcs[h][r][2 * j + 1];
              const float lo = v[hb * 4 + j], hi = v[hb * 4 + j + 2];
              v[hb * 4 + j] = lo * c - hi * sn;
              v[hb * 4 + j + 2] = hi * c + lo * sn;
            }
          }
        }
        T *C = (T *)g.C + (size_t)row * g.ldc + col0;
#pragma unroll
        for (int j = 0; j < NT; ++j) C[j * 16] = to_elem<T>(v[j]);
      } else if (EM == E_RESID) {
        float *C = (float *)g.C + (size_t)row * g.ldc + col0;
#pragma unroll
        for (int j = 0; j < NT; ++j) C[j * 16] = res[h][r][j] + v[j];
      } else if (EM == E_RELU) {
        T *C = (T *)g.C + (size_t)row * g.ldc + col0;
#pragma unroll
        for (int j = 0; j < NT; ++j) C[j * 16] = to_elem<T>(fmaxf(v[j], 0.f));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// attention: one block = up to 64 NSUB queries of one sequence and one head.
// S^T = K Q^T and O^T = V^T P^T keep each lane's 4 x 4 scores, its running
// max / sum and its output column on the same query (lane % 16).
// ---------------------------------------------------------------------------

// A fragment (8 elements per lane) through a buffer resource at byte offset voff.
template <typename T> __device__ inline Frag<T> ldb_frag(__amdgpu_buffer_rsrc_t r, int voff);
template <> __device__ inline Frag<bf16> ldb_frag<bf16>(__amdgpu_buffer_rsrc_t r, int voff) {
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
  return f;
}
template <> __device__ inline Frag<float> ldb_frag<float>(__amdgpu_buffer_rsrc_t r, int voff) {
  Frag<float> f;
  f.lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
  f.hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0));
  return f;
}

// Slot of key k (0..63) in the transposed V tile: the 8 keys that lane group
// g feeds to one 32-key step, {4g..4g+3, 16+4g..16+4g+3}, become contiguous.
__device__ inline int vt_slot(int k) {
  const int w = k & 31;
  return (k & 32) + ((w >> 2) & 3) * 8 + (w >> 4) * 4 + (w & 3);
}

// An empty instruction that reads the fragments: everything that produces
// them (loads in flight) must have completed here.  Emits no code.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline void frag_touch(const Frag<bf16> &a, const Frag<bf16> &b) {
  asm volatile("" ::"v"(__builtin_bit_cast(i32x4, a.v)), "v"(__builtin_bit_cast(i32x4, b.v)));
}
__device__ inline void frag_touch(const Frag<float> &a, const Frag<float> &b) {
  asm volatile("" ::"v"(a.lo), "v"(a.hi), "v"(b.lo), "v"(b.hi));
}

// V^T rows in LDS are swizzled in granules of 8 elements (one lane's operand
// read): granule q of row d sits at q ^ (2 ((d >> 4) & 3)).  The staging
// writes put 8 rows 8 apart into one instruction, which would otherwise land
// in the same banks (8-way); with the swizzle they are 2-way, the least this
// thread mapping allows, while the operand reads (16 consecutive rows, one
// swizzle value) stay conflict-free.
__device__ inline int vt_swz(int d, int slot) {
  return ((((slot >> 3) ^ (((d >> 4) & 3) << 1)) & 7) << 3) | (slot & 7);
}

// max of three / two floats with no NaN-quieting copies of the operands (the
// compiler's fmaxf first canonicalizes every operand that comes from a
// matrix-core result; scores are never signalling NaNs).
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Maximum over the four 16-lane rows of a wave for each lane position (lanes
// i, i + 16, i + 32, i + 48): the row-swap permutes pair rows 0-1 and 2-3,
// then the two halves, without a round trip through LDS.
__device__ inline float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = max2f(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return max2f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename T> __device__ inline Frag<T> ones_frag();
template <> __device__ inline Frag<bf16> ones_frag<bf16>() {
  Frag<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)1.0f;
  return f;
}
template <> __device__ inline Frag<float> ones_frag<float>() {
  return Frag<float>{f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}};
}

template <typename T>
__device__ inline void store_vt_pair(T *row, int slot, float a, float b);
template <>
__device__ inline void store_vt_pair<bf16>(bf16 *row, int slot, float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (bf16)a;
  p[1] = (bf16)b;
  *reinterpret_cast<bf16x2 *>(row + slot) = p;
}
template <>
__device__ inline void store_vt_pair<float>(float *row, int slot, float a, float b) {
  *reinterpret_cast<float2 *>(row + slot) = make_float2(a, b);
}

// NSUB query sub-tiles of 16 per wave, 4 waves: a block covers 64 NSUB
// queries.  Masking is evaluated only on key tiles that reach past the
// sequence end or, on local layers, past the window of some query.
//
// q arrives pre-scaled by log2(e) / sqrt(64) (the q rows of the projection
// weights and bias carry the factor, folded in at load), so scores are in the
// exp2 domain.  Each query keeps a reference maximum m; its score
// accumulators start at -m, so a probability is one exp2 of the accumulator,
// and the row sums l run on the matrix cores as a product with a ones
// fragment, from the same bf16 probabilities the P.V product uses.
//
// PF: key tiles in flight (register slots) on the rolling path, for grids of
// about one work-group per CU or less, where the registers cost no
// occupancy.  The marker rows' attention over a long sequence (8,192 keys)
// gains from it; a 1,024-key item at batch 1 does not, its one wave per SIMD
// being bound by the chain of each tile's own arithmetic.  The per-query
// arithmetic is the same for every PF and item size, so results do not
// depend on the batch.
template <typename T, int NSUB, bool kPre3 = false, int PF = 1>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  static_assert(PF >= 1 && (!kPre3 || PF == 1), "prefetch depth");
  // LDS row stride (elements): 80 makes the 16-byte operand reads (16 rows x
  // 4 chunks per 16 lanes) conflict-free on gfx950; 72 measured 2-way.
  constexpr int KS = 80;
  constexpr int QW = 16 * NSUB;
  __shared__ __attribute__((aligned(16))) T sK[2][64 * KS];
  __shared__ __attribute__((aligned(16))) T sV[2][64 * KS];  // [d][slot]
  const AttnWork w = a.work[a.rev ? gridDim.x - 1 - blockIdx.x : blockIdx.x];
  if (w.n_q <= 0) return;  // padding item of the XCD layout
  const int h = a.rev ? gridDim.y - 1 - blockIdx.y : blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15, g = lane >> 4;
  const bool local = a.half_window >= 0;
  const int W = a.half_window;

  Frag<T> fq[NSUB][2];
  int qpos[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int qi = wave * QW + 16 * s + ql;
    qpos[s] = w.q_pos0 + qi;
    const T *qp = (const T *)a.q + (size_t)(w.q_row0 + min(qi, w.n_q - 1)) * a.q_stride + h * kHeadDim;
    fq[s][0] = load_frag(qp + g * 8);
    fq[s][1] = load_frag(qp + 32 + g * 8);
  }

  int lo = 0, hi = w.kv_len;
  if (local) {
    lo = max(0, w.q_pos0 - W);
    hi = min(w.kv_len, w.q_pos0 + w.n_q + W);
  }
  const int n_tiles = (hi - lo + 63) >> 6;
  // key tiles [base, base + 64) inside every one of a wave's query windows need no mask
  // this wave's query positions (wave-uniform)
  const int wq0 = w.q_pos0 + __builtin_amdgcn_readfirstlane(wave) * QW, wq_last = wq0 + QW - 1;

  // K and V rows through buffer resources covering exactly this sequence's
  // rows: a row past its end reads as zeros (a masked key), so no load
  // clamps; the whole byte offset is per lane, where the range check sees it
  const int row_bytes = a.kv_stride * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>((const T *)a.k + (size_t)w.kv_row0 * a.kv_stride), (short)0, w.kv_len * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>((const T *)a.v + (size_t)w.kv_row0 * a.kv_stride), (short)0, w.kv_len * row_bytes, 0x00020000);
  const int colb = (h * kHeadDim + (tid & 7) * 8) * (int)sizeof(T);
  // this thread's rows of tile 0 (keys lo + tid / 8 and + 32; values
  // lo + 2 (tid / 8) and + 1); tile t is those rows + 64 t
  const int koff = (lo + (tid >> 3)) * row_bytes + colb, voff = (lo + 2 * (tid >> 3)) * row_bytes + colb;

  // a tile's K and V rows of this thread, in register slot r: kPre3 keeps
  // all (at most 3) tiles of a window item in flight from the start, the
  // rolling path PF tiles (tile t in slot t % PF)
  constexpr int NR = kPre3 ? 3 : PF;
  Frag<T> rk0[NR], rk1[NR], rv0[NR], rv1[NR];
  // No branch: a load under a branch leaves its register to be merged at
  // the join, and the compiler waits for the load there, not where the data
  // is first used.
  auto load_tile = [&](int t, int r) {
    const int to = t * 64 * row_bytes;
    rk0[r] = ldb_frag<T>(rsk, koff + to);
    rk1[r] = ldb_frag<T>(rsk, koff + to + 32 * row_bytes);
    rv0[r] = ldb_frag<T>(rsv, voff + to);
    rv1[r] = ldb_frag<T>(rsv, voff + to + row_bytes);
  };
  auto store_tile = [&](int buf, int r) {
    const int c = (tid & 7) * 8;
    store_frag(&sK[buf][(tid >> 3) * KS + c], rk0[r]);
    store_frag(&sK[buf][((tid >> 3) + 32) * KS + c], rk1[r]);
    const int slot = vt_swz(c, vt_slot(2 * (tid >> 3)));  // rows c .. c+7 share d >> 4
#pragma unroll
    for (int e = 0; e < 8; ++e) store_vt_pair<T>(&sV[buf][(c + e) * KS], slot, frag_get(rv0[r], e), frag_get(rv1[r], e));
  };

  // per query (lane % 16): the reference maximum m (the accumulators start at
  // -m), the growth threshold (-inf until the query's first key, then 8),
  // row sum and output
  float m[NSUB], thr[NSUB];
  f32x4 minit[NSUB], lsum[NSUB], o[NSUB][4];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    m[s] = 0.f;
    thr[s] = -INFINITY;
    minit[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const Frag<T> ones = ones_frag<T>();

  if (n_tiles <= 0) {  // no key (cannot happen for a valid work list): zero output
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int qi = wave * QW + 16 * s + ql;
      if (qi < w.n_q) {
        T *op = (T *)a.o + (size_t)(w.q_row0 + qi) * a.o_stride + h * kHeadDim + 4 * g;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
#pragma unroll
          for (int r = 0; r < 4; ++r) op[ds * 16 + r] = to_elem<T>(0.f);
      }
    }
    return;
  }
  // unconditional preamble: the first tile's stores wait for every earlier
  // load (the q fragments), so no wait for them is left inside the loop,
  // where it would also stall on the next tile's prefetch
  load_tile(0, 0);
  if constexpr (kPre3) {  // a window item meets at most 3 tiles; tiles beyond n_tiles are loaded and unused
    load_tile(1, 1);
    load_tile(2, 2);
  } else {
#pragma unroll
    for (int r = 1; r < PF; ++r) load_tile(r, r);  // likewise past the last tile
  }
  store_tile(0, 0);
  // the q fragments must have arrived before the loop: otherwise the
  // compiler places their wait at its first use inside the loop, where it
  // would also stall every iteration on the next tile's prefetch
#pragma unroll
  for (int s = 0; s < NSUB; ++s) frag_touch(fq[s][0], fq[s][1]);
  __syncthreads();
  // one 64-key tile from LDS buffer cur
  auto tile_step = [&](int t, int cur) {
    // S^T = K Q^T - m for each query sub-tile
    f32x4 sc[NSUB][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const T *kr = &sK[cur][(ks * 16 + ql) * KS + g * 8];
      const Frag<T> k0 = load_frag(kr), k1 = load_frag(kr + 32);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        sc[s][ks] = minit[s];
        mfma(sc[s][ks], k0, fq[s][0]);
        mfma(sc[s][ks], k1, fq[s][1]);
      }
    }
    const int base = lo + t * 64;
    const bool need_mask = base + 64 > hi || (local && (base < wq_last - W || base + 63 > wq0 + W));
    if (need_mask) {
      // allowed keys of a lane form one range: its j = 16 ks + r (key
      // base + 4 g + j) is allowed iff j - jlo <= span, unsigned
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int k0 = base + 4 * g;
        const int klo = local ? max(qpos[s] - W, 0) : 0;
        const int khi = local ? min(qpos[s] + W, hi - 1) : hi - 1;
        const int jlo = klo - k0;
        const unsigned span = (unsigned)(khi - klo);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((unsigned)(16 * ks + r - jlo) > span) sc[s][ks][r] = -INFINITY;
      }
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      // tile maximum relative to m: 16 values per lane, then across the 4 rows
      float mt = max2f(max3f(max3f(sc[s][0][0], sc[s][0][1], sc[s][0][2]), max3f(sc[s][0][3], sc[s][1][0], sc[s][1][1]),
                             max3f(sc[s][1][2], sc[s][1][3], sc[s][2][0])),
                       max3f(max3f(sc[s][2][1], sc[s][2][2], sc[s][2][3]), max3f(sc[s][3][0], sc[s][3][1], sc[s][3][2]),
                             sc[s][3][3]));
      mt = rows_max(mt);
      // Lazy rescale: m moves only when a tile's maximum exceeds it by more
      // than 8 (or on the query's first key), so probabilities stay <= 2^8;
      // the ratio o / l is unchanged.  Most tiles after the first need none.
      // Before the first key o and l are 0, and alpha is capped so that
      // 0 * alpha stays 0.
      const bool grow = mt > thr[s];
      if (__any(grow)) {
        const float delta = grow ? mt : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(fminf(-delta, 64.f));
        lsum[s] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[s][i] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sc[s][ks] -= delta;
        m[s] += delta;
        thr[s] = grow ? 8.f : thr[s];
        minit[s] = f32x4{-m[s], -m[s], -m[s], -m[s]};
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[s][ks][r] = __builtin_amdgcn_exp2f(sc[s][ks][r]);
    }
    // O^T += V^T P^T and l += 1 P^T
#pragma unroll
    for (int kstep = 0; kstep < 2; ++kstep) {
      Frag<T> fp[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        float pv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = sc[s][2 * kstep][r];
          pv[4 + r] = sc[s][2 * kstep + 1][r];
        }
        frag_from(fp[s], pv);
        mfma(lsum[s], ones, fp[s]);
      }
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const int d = ds * 16 + ql;
        const Frag<T> vf = load_frag(&sV[cur][d * KS + vt_swz(d, kstep * 32 + g * 8)]);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) mfma(o[s][ds], vf, fp[s]);
      }
    }
  };
  if constexpr (kPre3) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t < n_tiles) {
        tile_step(t, t & 1);
        if (t + 1 < n_tiles) store_tile((t + 1) & 1, t + 1);
        __syncthreads();
      }
    }
  } else {
    // slot t % PF: tile t reached LDS at the end of step t - 1 (or before the
    // loop), so step t refills the slot with tile t + PF (past the last tile:
    // loaded, never stored)
    for (int t0 = 0; t0 < n_tiles; t0 += PF) {
#pragma unroll
      for (int r = 0; r < PF; ++r) {
        const int t = t0 + r;
        if (t < n_tiles) {
          load_tile(t + PF, r);
          tile_step(t, t & 1);
          if (t + 1 < n_tiles) store_tile((t + 1) & 1, (r + 1) % PF);
          __syncthreads();
        }
      }
    }
  }
  // Output rows o / l.  bf16: each wave's 16 NSUB x 64 outputs go through its
  // own part of the K buffers (free after the last tile's barrier), 16-byte
  // chunks XOR-swizzled by row so that the reads are free of bank conflicts,
  // and leave as whole 128-byte rows of the head: 2 NSUB store instructions
  // per wave instead of 4 NSUB of 16 rows x 32 bytes.  FP32: straight from
  // the accumulators.
  if constexpr (sizeof(T) == 2) {
    T *st = &sK[0][0] + wave * (16 * NSUB * kHeadDim);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const float lt = lsum[s][0];  // every row of the ones product holds the query's sum
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const int rl = 16 * s + ql, sw = ql & 7;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)(o[s][ds][r] * inv);
        const int d0 = ds * 16 + 4 * g;
        *reinterpret_cast<bf16x4 *>(st + rl * kHeadDim + (((d0 >> 3) ^ sw) << 3) + (d0 & 7)) = v;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2 * NSUB; ++kk) {
      const int rl = 8 * kk + (lane >> 3), c = lane & 7, qi = wave * QW + rl;
      const bf16x8 v = *reinterpret_cast<const bf16x8 *>(st + rl * kHeadDim + ((c ^ (rl & 7)) << 3));
      if (qi < w.n_q)
        *reinterpret_cast<bf16x8 *>((T *)a.o + (size_t)(w.q_row0 + qi) * a.o_stride + h * kHeadDim + 8 * c) = v;
    }
  } else {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const float lt = lsum[s][0];
      const int qi = wave * QW + 16 * s + ql;
      if (qi < w.n_q) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        T *op = (T *)a.o + (size_t)(w.q_row0 + qi) * a.o_stride + h * kHeadDim + 4 * g;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
#pragma unroll
          for (int r = 0; r < 4; ++r) op[ds * 16 + r] = to_elem<T>(o[s][ds][r] * inv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// row kernels
// ---------------------------------------------------------------------------

// h = LayerNorm(x; gain) + type_rows[qtype of the token's sequence]; h may alias x.
__global__ __launch_bounds__(256) void final_ln_type_kernel(const float *x, const float *__restrict__ gain,
                                                            const float *__restrict__ type_rows,
                                                            const int *__restrict__ qtype,
                                                            const int *__restrict__ tok_seq, int T, float *h) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *xr = x + (size_t)t * kWidth;
  float v[6], s = 0.f;
#pragma unroll
  for (int i = 0; i < 6; ++i) { v[i] = xr[lane + 64 * i]; s += v[i]; }
  const float mean = wave_sum(s) * (1.0f / kWidth);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 6; ++i) { const float d = v[i] - mean; q += d * d; }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / kWidth) + kLnEps);
  const float *tr = type_rows + (size_t)qtype[tok_seq[t]] * kWidth;
  float *hr = h + (size_t)t * kWidth;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int c = lane + 64 * i;
    hr[c] = (v[i] - mean) * rstd * gain[c] + tr[c];
  }
}

// out[t] = LayerNorm(x[t]; gain, shift) as the GEMM element type; gain == nullptr
// copies x unchanged (the first layer's identity pre-norm).  One row per
// 16-lane row of the wave (lane j: columns 64 c + 4 j .. + 3), with the
// statistics and arithmetic of the GEMM's fused LayerNorm (ln_row16), so both
// give identical operands.
template <typename T>
__global__ __launch_bounds__(256) void ln_rows_kernel(const float *__restrict__ x, const float *__restrict__ gain,
                                                      const float *__restrict__ shift, int n, T *__restrict__ out) {
  const int lj = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= n) return;  // whole 16-lane rows leave together
  f32x4 y[6];
  const float *xr = x + (size_t)t * kWidth + 4 * lj;
#pragma unroll
  for (int c = 0; c < 6; ++c) y[c] = *reinterpret_cast<const f32x4 *>(xr + 64 * c);
  if (gain != nullptr) {
    float mean, rstd;
    ln_row16(y, mean, rstd);
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(gain + 64 * c + 4 * lj);
      f32x4 sh = f32x4{0.f, 0.f, 0.f, 0.f};  // absent shift: + 0, as in the GEMM's fused LayerNorm
      if (shift) sh = *reinterpret_cast<const f32x4 *>(shift + 64 * c + 4 * lj);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[c][e] = (y[c][e] - mean) * rstd * gm[e] + sh[e];
    }
  }
  T *o = out + (size_t)t * kWidth + 4 * lj;
#pragma unroll
  for (int c = 0; c < 6; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[64 * c + e] = to_elem<T>(y[c][e]);
}

// dst[m] = src[rows[m]] (the marker rows); block 0 also clears the scorer's
// counters of this pass (cnt[0, n_cnt)), which score_kernel leaves cleared.
__global__ __launch_bounds__(256) void gather_rows_kernel(const float *__restrict__ src,
                                                          const int *__restrict__ rows, int n,
                                                          float *__restrict__ dst, int *__restrict__ cnt,
                                                          int n_cnt) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_cnt; i += 256) cnt[i] = 0;
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= n) return;
  const float *s = src + (size_t)rows[m] * kWidth;
  float *d = dst + (size_t)m * kWidth;
#pragma unroll
  for (int i = 0; i < 6; ++i) d[lane + 64 * i] = s[lane + 64 * i];
}

// The scorer on the marker rows, FP32 in every mode: logit = w2 . GELU(W1 .
// LayerNorm(z; g, b) + b1) + b2, one launch.  Block (rb, cb) takes rows
// 16 rb .. 16 rb + 15 and hidden columns 64 cb .. 64 cb + 63: the rows are
// normalized into LDS (the LayerNorm kernel's thread mapping and arithmetic),
// wave w forms 16 hidden columns on the FP32 matrix cores (A = W1 rows, B =
// the normalized rows; lane l feeds k = 4 (l / 16) + q of each 16-k block to
// product q), adds b1, applies GELU and its part of the dot product; the
// block's share of each row's logit goes to part[row][cb].  The last of the
// kScoreBlocks blocks of a row group to finish (counted in cnt[rb]) adds the
// shares in order of cb, plus b2, and clears cnt[rb] again.
constexpr int kScoreBlocks = kWidth / 64;
__global__ __launch_bounds__(256) void score_kernel(const float *__restrict__ z, const float *__restrict__ g,
                                                    const float *__restrict__ b, const float *__restrict__ W1,
                                                    const float *__restrict__ b1, const float *__restrict__ w2,
                                                    const float *__restrict__ b2, int M, float *part, int *cnt,
                                                    float *__restrict__ logits, int rev) {
  __shared__ __attribute__((aligned(16))) float sU[16][kWidth + 4];  // 4 spare: conflict-free operand reads
  __shared__ float sP[4][16];
  __shared__ int sLast;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = rev ? gridDim.x - 1 - blockIdx.x : blockIdx.x, cb = rev ? gridDim.y - 1 - blockIdx.y : blockIdx.y;
  const int lj = lane & 15, lr = lane >> 4;
  // this lane's W1 operands (row 64 cb + 16 w + lj, k = 16 i + 4 lr .. + 3)
  // and epilogue columns, all in flight during the LayerNorm
  constexpr int KB = kWidth / 16;
  f32x4 wa[KB];
  const float *wr = W1 + (size_t)(64 * cb + 16 * wave + lj) * kWidth + 4 * lr;
#pragma unroll
  for (int i = 0; i < KB; ++i) wa[i] = *reinterpret_cast<const f32x4 *>(wr + 16 * i);
  const int hc0 = 64 * cb + 16 * wave + 4 * lr;
  const f32x4 bias1 = *reinterpret_cast<const f32x4 *>(b1 + hc0), wout = *reinterpret_cast<const f32x4 *>(w2 + hc0);
  {
    const int lr16 = tid & 15, rl = tid >> 4;
    const float *xr = z + (size_t)min(16 * rb + rl, M - 1) * kWidth + 4 * lr16;
    f32x4 y[6];
#pragma unroll
    for (int c = 0; c < 6; ++c) y[c] = *reinterpret_cast<const f32x4 *>(xr + 64 * c);
    float mean, rstd;
    ln_row16(y, mean, rstd);
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(g + 64 * c + 4 * lr16);
      const f32x4 sh = *reinterpret_cast<const f32x4 *>(b + 64 * c + 4 * lr16);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[c][e] = (y[c][e] - mean) * rstd * gm[e] + sh[e];
      *reinterpret_cast<f32x4 *>(&sU[rl][64 * c + 4 * lr16]) = y[c];
    }
  }
  __syncthreads();
  const float *ur = &sU[lj][4 * lr];
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const f32x4 u = *reinterpret_cast<const f32x4 *>(ur + 16 * i);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[i][q], u[q], acc, 0, 0, 0);
  }
  // lane l holds hidden columns 64 cb + 16 w + 4 lr + r of row lj
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) s += gelu_erf(acc[r] + bias1[r]) * wout[r];
  {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  if (lr == 0) sP[wave][lj] = s;
  __syncthreads();
  const int row = 16 * rb + tid;
  if (tid < 16 && row < M) part[(size_t)row * kScoreBlocks + cb] = ((sP[0][tid] + sP[1][tid]) + sP[2][tid]) + sP[3][tid];
  __threadfence();  // this block's shares, visible device-wide before its count
  __syncthreads();
  if (tid == 0) sLast = atomicAdd(&cnt[rb], 1) == kScoreBlocks - 1;
  __syncthreads();
  if (!sLast) return;
  __threadfence();  // every other block's shares, after their counts
  if (tid < 16 && row < M) {
    const float *pr = part + (size_t)row * kScoreBlocks;
    float t = pr[0];
#pragma unroll
    for (int c = 1; c < kScoreBlocks; ++c) t += pr[c];
    logits[row] = t + b2[0];
  }
  if (tid == 0) cnt[rb] = 0;
}

// One wave per question: softmax over its options and the three read-offs.
__global__ __launch_bounds__(256) void probs_kernel(const float *__restrict__ logits,
                                                    const int *__restrict__ marker_offsets,
                                                    const int *__restrict__ qtype, int n_seqs,
                                                    float *probs, float *answer, int *argmax,
                                                    float *maxprob) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n_seqs) return;
  const int first = marker_offsets[b], n = marker_offsets[b + 1] - first;
  const bool on = lane < n;
  const float v = on ? logits[first + lane] : -INFINITY;
  const float mx = wave_max(v);
  const float e = on ? expf(v - mx) : 0.f;
  const float sum = wave_sum(e);
  const float p = e / sum;
  // first index holding the maximum
  int idx = (on && v == mx) ? lane : 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) idx = min(idx, __shfl_xor(idx, o, 64));
  const float expect = wave_sum(on ? (float)lane * p : 0.f);
  const float p1 = __shfl(p, 1, 64);
  if (on && probs) probs[first + lane] = p;
  if (lane == 0) {
    const int qt = qtype[b];
    if (answer) answer[b] = qt == 0 ? (float)idx : (qt == 1 ? expect : p1);
    if (argmax) argmax[b] = idx;
    if (maxprob) maxprob[b] = 1.0f / sum;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_embed(const int32_t *ids, const float *emb, const float *gain, int T,
                        const int *seq_offsets, int n_seqs, float *x, int *pos, int *tok_seq,
                        hipStream_t s) {
  if (T <= 0) return hipSuccess;
  embed_kernel<<<(T + 3) / 4, 256, 0, s>>>(ids, emb, gain, T, seq_offsets, n_seqs, x, pos, tok_seq);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int NS, bool LNA = false, int KFIX = 0, bool RF = false, bool F8 = false>
static hipError_t gemm_dispatch(int emode, const GemmArgs &a, hipStream_t s) {
  const int tiles_n = a.N / BN, n_tiles = ((a.M + BM - 1) / BM) * tiles_n;
  constexpr bool pairs = (BN / 32) % 4 == 0;  // 64-column groups per wave: GEGLU and RoPE epilogues
  switch (emode) {
    case E_STORE:
      if constexpr (!pairs) return hipErrorInvalidValue;
      else gemm_kernel<T, BM, BN, E_STORE, NS, LNA, KFIX, RF, F8><<<n_tiles, 256, 0, s>>>(a, tiles_n, n_tiles);
      break;
    case E_GEGLU:
      if constexpr (!pairs || (LNA && !RF)) return hipErrorInvalidValue;
      else gemm_kernel<T, BM, BN, E_GEGLU, NS, LNA, KFIX, RF, F8><<<n_tiles, 256, 0, s>>>(a, tiles_n, n_tiles);
      break;
    case E_RELU:
      if constexpr ((LNA && !RF) || F8) return hipErrorInvalidValue;
      else gemm_kernel<T, BM, BN, E_RELU, NS, LNA, KFIX, RF><<<n_tiles, 256, 0, s>>>(a, tiles_n, n_tiles);
      break;
    case E_RESID:
      if constexpr (LNA || RF || F8) return hipErrorInvalidValue;
      else gemm_kernel<T, BM, BN, E_RESID, NS, false, KFIX><<<n_tiles, 256, 0, s>>>(a, tiles_n, n_tiles);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile choice: the largest M tile that still gives at least one tile per CU;
// grids of at most one tile per CU take the deep pipeline below.
hipError_t launch_gemm(bool bf16_mode, int emode, const GemmArgs &a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.N % 128 != 0 || a.K % 64 != 0) return hipErrorInvalidValue;
  const long nt = a.N / 128;
  if (bf16_mode) {
    if (((a.M + 255) / 256) * nt >= 256) return gemm_dispatch<bf16, 256, 128, 2>(emode, a, s);
    if (((a.M + 127) / 128) * nt >= 256) return gemm_dispatch<bf16, 128, 128, 2>(emode, a, s);
    if (((a.M + 63) / 64) * nt > 256) return gemm_dispatch<bf16, 64, 128, 2>(emode, a, s);
    // One round of work-groups: the model's K values get a fully unrolled K
    // loop.  Such a grid is bound by each work-group's own memory round trip
    // and by what one CU can take in, so a residual update (N = 384) takes
    // the smallest tile that still fits the CUs in one round: 32 x 64 moves
    // (32 + 64) K elements per work-group against 192 K for 64 x 128.
    if (emode == E_RESID && a.N % 64 == 0) {
      const long t32 = ((a.M + 31) / 32) * (a.N / 64), t64 = ((a.M + 63) / 64) * (a.N / 64);
      if (t32 <= 256 || t64 <= 256) {
        const bool r32 = t32 <= 256;
        switch (a.K) {
          case kWidth:
            return r32 ? gemm_dispatch<bf16, 32, 64, 6, false, kWidth>(emode, a, s)
                       : gemm_dispatch<bf16, 64, 64, 6, false, kWidth>(emode, a, s);
          case kGeglu:
            return r32 ? gemm_dispatch<bf16, 32, 64, 6, false, kGeglu>(emode, a, s)
                       : gemm_dispatch<bf16, 64, 64, 6, false, kGeglu>(emode, a, s);
          case kHeadFfn:
            return r32 ? gemm_dispatch<bf16, 32, 64, 6, false, kHeadFfn>(emode, a, s)
                       : gemm_dispatch<bf16, 64, 64, 6, false, kHeadFfn>(emode, a, s);
          default: break;
        }
      }
    }
    switch (a.K) {
      case kWidth: return gemm_dispatch<bf16, 64, 128, 6, false, kWidth>(emode, a, s);
      case kGeglu: return gemm_dispatch<bf16, 64, 128, 6, false, kGeglu>(emode, a, s);
      case kHeadFfn: return gemm_dispatch<bf16, 64, 128, 6, false, kHeadFfn>(emode, a, s);
      default: return gemm_dispatch<bf16, 64, 128, 6>(emode, a, s);
    }
  }
  if (((a.M + 127) / 128) * nt >= 256) return gemm_dispatch<float, 128, 128, 2>(emode, a, s);
  if (((a.M + 63) / 64) * nt <= 256) {
    switch (a.K) {
      case kWidth: return gemm_dispatch<float, 64, 128, 5, false, kWidth>(emode, a, s);
      case kGeglu: return gemm_dispatch<float, 64, 128, 5, false, kGeglu>(emode, a, s);
      case kHeadFfn: return gemm_dispatch<float, 64, 128, 5, false, kHeadFfn>(emode, a, s);
      default: break;
    }
  }
  return gemm_dispatch<float, 64, 128, 2>(emode, a, s);
}

hipError_t launch_ln_gemm(bool bf16_mode, int emode, const GemmArgs &a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.N % 128 != 0 || a.K != kWidth || !a.ln_x) return hipErrorInvalidValue;
  const long nt = a.N / 128, tiles64 = ((a.M + 63) / 64) * nt;
  // e4m3 products: every batch size, all 6 weight stages up front; 64 x 128
  // tiles (72 KB of LDS: two work-groups per CU), or 64 x 256 when 128
  // columns would need a second round and 256 fit the CUs in one
  if (a.w_scale != nullptr) {
    if (!bf16_mode || a.ln_gain == nullptr || (emode != E_STORE && emode != E_GEGLU)) return hipErrorInvalidValue;
    if (emode == E_GEGLU && tiles64 > 256 && a.N % 256 == 0 && ((a.M + 63) / 64) * (a.N / 256) <= 256)
      return gemm_dispatch<bf16, 64, 256, 6, true, 0, true, true>(emode, a, s);
    return gemm_dispatch<bf16, 64, 128, 6, true, 0, true, true>(emode, a, s);
  }
  // the GEMM alone would take 64-row tiles: normalize inside it
  // (the GEGLU and ReLU products normalize unconditionally inside: they need a gain)
  if (bf16_mode && (emode == E_STORE || ((emode == E_GEGLU || emode == E_RELU) && a.ln_gain != nullptr)) &&
      ((a.M + 127) / 128) * nt < 256) {
    // one round of work-groups (1 per CU: 144 KB of LDS): 6 stages of a
    // 128-column tile, or 3 of a 256-column tile when 128 would need two
    // with a gain the rows are loaded (and normalized) ahead of the weights
    const bool rf = a.ln_gain != nullptr;
    if (tiles64 <= 256)
      return rf ? gemm_dispatch<bf16, 64, 128, 6, true, 0, true>(emode, a, s)
                : gemm_dispatch<bf16, 64, 128, 6, true>(emode, a, s);
    if (a.N % 256 == 0 && ((a.M + 63) / 64) * (a.N / 256) <= 256)
      return rf ? gemm_dispatch<bf16, 64, 256, 3, true, 0, true>(emode, a, s)
                : gemm_dispatch<bf16, 64, 256, 3, true>(emode, a, s);
    return rf ? gemm_dispatch<bf16, 64, 128, 2, true, 0, true>(emode, a, s)
              : gemm_dispatch<bf16, 64, 128, 2, true>(emode, a, s);
  }
  hipError_t e = launch_ln_rows(bf16_mode, a.ln_x, a.ln_gain, a.ln_shift, a.M, const_cast<void *>(a.A), s);
  if (e != hipSuccess) return e;
  return launch_gemm(bf16_mode, emode, a, s);
}

hipError_t launch_ln_rows(bool bf16_out, const float *x, const float *gain, const float *shift, int n, void *out,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (bf16_out) ln_rows_kernel<bf16><<<(n + 15) / 16, 256, 0, s>>>(x, gain, shift, n, (bf16 *)out);
  else ln_rows_kernel<float><<<(n + 15) / 16, 256, 0, s>>>(x, gain, shift, n, (float *)out);
  return hipGetLastError();
}

hipError_t launch_attention(bool bf16_mode, const AttnArgs &a, int n_work, int queries_per_block, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work, kHeads);
  if (queries_per_block == 64) {
    // a window item (64 queries, +-64 keys) meets at most 3 key tiles: all in
    // flight from the start.  Whole-sequence 64-query items run on grids of at
    // most about one work-group per CU (small batches, marker rows): 3 tiles
    // in flight.
    const bool pre3 = a.half_window >= 0 && a.half_window <= kHalfWindow;
    if (bf16_mode) {
      if (pre3) attn_kernel<bf16, 1, true><<<grid, 256, 0, s>>>(a);
      else attn_kernel<bf16, 1, false, 3><<<grid, 256, 0, s>>>(a);
    } else {
      attn_kernel<float, 1><<<grid, 256, 0, s>>>(a);
    }
  } else if (queries_per_block == 128) {
    if (bf16_mode) attn_kernel<bf16, 2><<<grid, 256, 0, s>>>(a);
    else attn_kernel<float, 2><<<grid, 256, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_final_ln_type(const float *x, const float *gain, const float *type_rows,
                                const int *qtype, const int *tok_seq, int T, float *h, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  final_ln_type_kernel<<<(T + 3) / 4, 256, 0, s>>>(x, gain, type_rows, qtype, tok_seq, T, h);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const float *src, const int *rows, int n, float *dst, int *score_cnt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  gather_rows_kernel<<<(n + 3) / 4, 256, 0, s>>>(src, rows, n, dst, score_cnt, score_groups(n));
  return hipGetLastError();
}

hipError_t launch_score(const float *z, const float *g, const float *b, const float *W1, const float *b1,
                        const float *w2, const float *b2, int n, float *part, int *cnt, float *logits, int rev,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  score_kernel<<<dim3(score_groups(n), kScoreBlocks), 256, 0, s>>>(z, g, b, W1, b1, w2, b2, n, part, cnt, logits,
                                                                    rev);
  return hipGetLastError();
}

hipError_t launch_probs(const float *logits, const int *marker_offsets, const int *qtype, int n_seqs,
                        float *probs, float *answer, int *argmax, float *maxprob, hipStream_t s) {
  if (n_seqs <= 0) return hipSuccess;
  probs_kernel<<<(n_seqs + 3) / 4, 256, 0, s>>>(logits, marker_offsets, qtype, n_seqs, probs, answer,
                                                argmax, maxprob);
  return hipGetLastError();
}

}  // namespace jl
