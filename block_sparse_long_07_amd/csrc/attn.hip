// Main Branch: exact softmax attention restricted to the selected KV blocks,
// organised KV-outer ("outer gather Q") [pnsm, section 7; yhxrc, 二;
// yololab, "KV Outer Gather Q是什麼？"].
//
// Prefill has two passes. Blocks selected by many queries of a 16-query unit
// (the query's own block, sink-like or planted blocks, blocks a local run of
// queries agrees on) are computed query-stationary: for each (unit, group) a
// workgroup of a persistent grid keeps the 16 queries' Q and running softmax
// state in registers and streams the unit's listed blocks through LDS,
// masking the rows that did not select a block (k_attn_dense). Every other (query, block) pair goes KV-outer: a
// persistent grid drains the tile queue built by the reverse index, a tile being
// (group g, KV block b, up to 16 queries that selected b); the block is staged
// once and each wave gathers the 16 query heads of a query (4 KiB, contiguous in
// the [N, Hq, d] layout) (k_attn_prefill). Both compute, on MFMA 16x16x32 bf16,
//   S^T (128 keys x 16 heads) = K_b (128 x 128) . Q^T        (32 MFMA)
//   P^T = 2^(S^T * scale*log2e - m),  l = sum P, per head
//   O^T (128 d x 16 heads)  += V_b^T (128 x 128 keys) . P^T  (32 MFMA)
// The S^T orientation puts one head's scores in one lane column, so softmax
// reductions are in-lane plus two cross-lane steps, and the P^T accumulator
// fragments feed the second contraction directly as its B operand (the key
// order inside a 32-key step is permuted identically in V^T's A operand).
// KV-outer outputs one softmax partial per (query, head, selected slot), o/l
// rounded to bf16 plus lse2 = m*c + log2(l); the dense pass, which runs after
// it, merges them with its own state without atomics (two-phase combine
// [pnsm, section 7]). Causal masking is needed only in the query's own block.
//
// K_b and V_b travel HBM -> LDS by direct LDS loads (global_load_lds, 16 bytes
// per lane, no registers), double-buffered so the next block streams in while
// the current one is computed. Both stay row-major in LDS (256 B per key row);
// the V^T operand is read with the transposing ds_read_b64_tr_b16. XOR
// swizzles of the 16-byte (K) and 32-byte (V) chunks keep the operand reads
// free of bank conflicts.
//
// Decode: one workgroup per (sequence, group) streams the selected blocks
// through LDS; one wave keeps the 16 heads' online softmax across them.
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"
#include "topk_row.h"

namespace msa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;
// LDS byte pointers (lds_char) stay in the local address space (32-bit
// addressing, no generic-pointer checks)

constexpr int kStage = 65536;  // bytes per staged block: K then V, 128 rows x 256 B each
constexpr int kVOff = 32768;

// Issue the direct-to-LDS loads of ROWS key rows of K and V (rows key0..,
// row stride `rstride` elements) into one stage: K at the stage start, V at
// VOFF. Slot s (16 B) of the K part holds row s/16, chunk (s%16) ^ (row & 15);
// of the V part, row s/16, 32-byte chunk ((s%16)/2) ^ (row & 7), half (s%2).
// Rows at or past `nvalid` repeat the last valid row, so every staged value is
// finite (those keys are masked).
template <int ROWS, int VOFF>
__device__ __forceinline__ void stage_rows(lds_char* stage, const uint16_t* kr0, const uint16_t* vr0,
                                           int64_t rstride, int nvalid, int wave, int nwaves) {
  const int lane = threadIdx.x & 63;
  for (int s0 = wave * 64; s0 < ROWS * 16; s0 += nwaves * 64) {
    const int slot = s0 + lane;
    const int r = slot >> 4, p = slot & 15;
    const int64_t row = (int64_t)min(r, nvalid - 1) * rstride;
    const int ck = p ^ (r & 15);
    const int cv = (((p >> 1) ^ (r & 7)) << 1) | (p & 1);
    lds_dma16(kr0 + row + ck * 8, stage + s0 * 16);
    lds_dma16(vr0 + row + cv * 8, stage + VOFF + s0 * 16);
  }
}

// Per-lane byte offsets of a wave's staging loads, the same for every block:
// slot s = 64*wave + lane of the layout above. A wave's next slots (64*nwaves
// further) are 4*nwaves rows further with the same swizzle when nwaves is a
// multiple of 4, so only the (uniform) base moves.
struct StageOffsets {
  uint32_t k, v;
};

__device__ __forceinline__ StageOffsets stage_offsets(int64_t rstride, int wave) {
  const int s = wave * 64 + (threadIdx.x & 63);
  const int r = s >> 4, p = s & 15;
  const int ck = p ^ (r & 15);
  const int cv = (((p >> 1) ^ (r & 7)) << 1) | (p & 1);
  return {(uint32_t)(((int64_t)r * rstride + ck * 8) * 2), (uint32_t)(((int64_t)r * rstride + cv * 8) * 2)};
}

// Element offset of key block b (of bk keys), group g in a [tokens][G][128] K
// or V array, from 32-bit uniform ints (blocks * bk * G stays below 2^31).
__device__ __forceinline__ uint64_t block_elems(int b, int bk, int G, int g) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(b * bk * G + g) * kHeadDim;
}

// A whole block (128 keys) per stage. A full block is loaded from uniform
// bases and the precomputed offsets (nwaves a multiple of 4); a partial one
// (the sequence's last) clamps its rows.
__device__ __forceinline__ void stage_block(lds_char* stage, const uint16_t* kr0, const uint16_t* vr0,
                                            int64_t rstride, int nvalid, int wave, int nwaves,
                                            const StageOffsets& off) {
  if (nvalid < kBlock) {
    stage_rows<kBlock, kVOff>(stage, kr0, vr0, rstride, nvalid, wave, nwaves);
    return;
  }
  const int64_t rows_it = (int64_t)4 * nwaves * rstride;  // elements per iteration
  for (int it = 0; it * 4 * nwaves < kBlock; ++it) {
    const int s0 = wave * 64 + it * nwaves * 64;
    lds_dma16_s(kr0 + it * rows_it, off.k, stage + s0 * 16);
    lds_dma16_s(vr0 + it * rows_it, off.v, stage + kVOff + s0 * 16);
  }
}

// A block of BK keys (BK < 128: the first BK rows of the stage; the layout of
// those rows is the one above).
template <int BK>
__device__ __forceinline__ void stage_block_bk(lds_char* stage, const uint16_t* kr0, const uint16_t* vr0,
                                               int64_t rstride, int nvalid, int wave, int nwaves,
                                               const StageOffsets& off) {
  if constexpr (BK == kBlock)
    stage_block(stage, kr0, vr0, rstride, nvalid, wave, nwaves, off);
  else
    stage_rows<BK, kVOff>(stage, kr0, vr0, rstride, nvalid, wave, nwaves);
}

__device__ __forceinline__ void wait_loads() { wait_vmcnt0(); }

// K A-operand of key tile t, d-step st: lane (c, qd) holds K[16t + c][32st + 8qd .. +7].
__device__ __forceinline__ bf16x8 lds_k(const lds_char* stage, int t, int st, int c, int qd) {
  const int p = (4 * st + qd) ^ c;  // (16t + c) & 15 == c
  const u32x4 v = *(const lds_u32x4*)(stage + (16 * t + c) * 256 + p * 16);
  return as_bf16x8(v);
}

// V^T A-operand of d-tile dt, key step st: lane (c, qd) holds V[kappa][16dt + c]
// for kappa = 32st + 4qd + {0..3} and 32st + 16 + 4qd + {0..3}. Each transposing
// read gives lane j of a 16-lane group element (4r + j/4, j%4) of the 16 x 4
// matrix whose row i is the 4 elements addressed by lane i; lane i therefore
// addresses row 32st + 4qd + i/4 (+16), dims 16dt + 4(i%4) .. +3.
template <int VOFF>
__device__ __forceinline__ bf16x8 lds_vt(const lds_char* stage, int dt, int st, int c, int qd) {
  const lds_char* vb = stage + VOFF;
  const int r1 = 32 * st + 4 * qd + (c >> 2), r2 = r1 + 16;
  const int off = 8 * (c & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + r1 * 256 + ((dt ^ (r1 & 7)) << 5) + off));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + r2 * 256 + ((dt ^ (r2 & 7)) << 5) + off));
  return as_bf16x8((u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                           __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
}

// Per-wave state of QN queries (16 heads each) against staged blocks.
//   qop: Q^T B-operands (4 steps over d); o[0..7]: O^T accumulators (head =
//   lane & 15, d = 16*dt + 4*(lane/16) + r); o[8]: every element is the softmax
//   denominator of the lane's head (see attend_block); m: reference max of the
//   raw scores per head.
template <int QN>
struct QueryGroup {
  static constexpr int kQN = QN;
  bf16x8 qop[QN][4];
  f32x4 o[QN][9];
  float m[QN];
};

// Vector memory instructions load_q issues (one 16-byte load per d-step, at
// per-lane addresses: always vector loads), for callers that wait on a
// counted vmcnt.
constexpr int kLoadQOps = 4;
template <class QG>
__device__ __forceinline__ void load_q(QG& qg, int n, const uint16_t* qrow) {
#pragma unroll
  for (int st = 0; st < kLoadQOps; ++st) qg.qop[n][st] = as_bf16x8(ld16(qrow + 32 * st));
}

// Running state before the first block: reference max -inf, zero accumulators.
template <class QG>
__device__ __forceinline__ void reset_state(QG& qg) {
#pragma unroll
  for (int n = 0; n < QG::kQN; ++n) {
    qg.m[n] = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 9; ++t) qg.o[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

// Instruction classes of the scheduling hints (sched_group_barrier masks).
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

// K operands of the first two d-steps of the first half of a staged block
// (key tiles 0..3): read as one batch, as early as the caller can, so their
// latency overlaps other work. The last two d-steps are read when the
// contraction starts.
constexpr int kPreSteps = 2;
struct KHalf {
  bf16x8 a[kPreSteps][4];  // [d-step][key tile]
};

__device__ __forceinline__ void load_k_half(KHalf& kh, const lds_char* stage) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
#pragma unroll
  for (int st = 0; st < kPreSteps; ++st)
#pragma unroll
    for (int t = 0; t < 4; ++t) kh.a[st][t] = lds_k(stage, t, st, c, qd);
}

// S^T = K_b . Q^T for key tiles 0..3, the first d-steps from preloaded operands.
template <int QN>
__device__ __forceinline__ void qk_half0(f32x4 (&s)[QN][4], const bf16x8 (&qop)[QN][4], const KHalf& kh,
                                         const lds_char* stage) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  bf16x8 a[4 - kPreSteps][4];
#pragma unroll
  for (int st = kPreSteps; st < 4; ++st)
#pragma unroll
    for (int t = 0; t < 4; ++t) a[st - kPreSteps][t] = lds_k(stage, t, st, c, qd);
#pragma unroll
  for (int n = 0; n < QN; ++n)
#pragma unroll
    for (int t = 0; t < 4; ++t) s[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // d-step outer, key tile inner: 4*QN independent accumulators between two
  // dependent MFMAs
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int n = 0; n < QN; ++n)
        s[n][t] = mfma16x16x32(st < kPreSteps ? kh.a[st][t] : a[st - kPreSteps][t], qop[n][st], s[n][t]);
}

// Causal mask of half h (MASKED: keys with index > lim[n] get -inf) and the
// max of each head's raw scores over the half, reduced over the lane groups.
template <bool MASKED, int QN>
__device__ __forceinline__ void half_max(f32x4 (&s)[QN][4], const int* lim, int h, float (&mx)[QN]) {
  const int qd = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int n = 0; n < QN; ++n) {
    if (MASKED) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * (4 * h + t) + 4 * qd + r > lim[n]) s[n][t][r] = -__builtin_inff();
    }
    float x = fmaxf(s[n][0][0], s[n][0][1]);
    x = fmaxf(fmaxf(x, s[n][0][2]), s[n][0][3]);
#pragma unroll
    for (int t = 1; t < 4; ++t) {
      x = fmaxf(fmaxf(x, s[n][t][0]), s[n][t][1]);
      x = fmaxf(fmaxf(x, s[n][t][2]), s[n][t][3]);
    }
    mx[n] = max_lane_groups(x);
  }
}

// p *= alpha[n] on packed bf16 operands (round to nearest even).
template <int QN>
__device__ __forceinline__ void scale_p(bf16x8 (&p)[QN][2], const float (&alpha)[QN]) {
#pragma unroll
  for (int n = 0; n < QN; ++n)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 w = __builtin_bit_cast(u32x4, p[n][j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(bf2f(w[i] & 0xffffu) * alpha[n], bf2f(w[i] >> 16) * alpha[n]);
      p[n][j] = as_bf16x8(w);
    }
}

// Exponent headroom of the lazily rescaled softmax: P may reach 2^kLazy
// before the running state is rescaled to a new reference max.
constexpr float kLazy = 8.0f;

// One exponential unit: P^T operand j of query n from scores s (half layout).
template <int QN>
__device__ __forceinline__ void exp_unit(const f32x4 (&s)[QN][4], const float (&mc)[QN], float scale_log2,
                                         bf16x8 (&p)[QN][2], int n, int j) {
  float e[8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      e[4 * u + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][2 * j + u][r], scale_log2, -mc[n]));
  p[n][j] = as_bf16x8((u32x4){pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                              pack_bf16x2(e[6], e[7])});
}

// Scheduling pattern of one pipelined region: NM MFMAs, NV VALU and ND LDS
// reads spread evenly between them; nothing moves across the region's end.
template <int NM, int NV, int ND, int I = 0>
__device__ __forceinline__ void sched_region() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    constexpr int vi = (NV * (I + 1)) / NM - (NV * I) / NM;
    constexpr int di = (ND * (I + 1)) / NM - (ND * I) / NM;
    if constexpr (vi > 0) __builtin_amdgcn_sched_group_barrier(kSchedValu, vi, 0);
    if constexpr (di > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, di, 0);
    sched_region<NM, NV, ND, I + 1>();
  } else {
    __builtin_amdgcn_sched_barrier(0);
  }
}

// f(integral_constant<int, I>) for I = B .. E-1, in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Online-softmax update of the running state with one staged block of 8 key
// tiles (V at VOFF): S^T = K_b . Q^T, p = 2^(s*c - m*c) with the logit scale
// folded into the exponent (c = scale * log2 e, reference max m kept on raw
// scores), O^T += V^T . P^T. The block is processed as two halves of four
// tiles, software-pipelined so that the VALU work of one half runs between
// the MFMAs of the other:
//   S0;  mask+max 0;  [S1 | exp 0];  mask+max 1;  [PV0 | exp 1];  PV1.
// In the pipelined parts every d-step (S1) or key step (PV) is a scheduling
// region of its own that also issues the operand reads of the next step.
//  * FIRST: fresh state; m is the first half's max and the accumulators start
//    at 0. Otherwise the state is rescaled only when some head's max exceeds
//    its reference by more than kLazy/c; the rescale is exact (every term is
//    multiplied by the same 2^((m_old - m_new) c)). A rescale decided by half
//    1 also scales the packed P of half 0, whose PV has not been issued yet.
//  * MASKED: the queries' own block; keys with index > lim[n] are masked. A
//    half whose keys are all masked leaves the state unchanged (its max is
//    -inf); key 0 of the own block is never masked.
//  * skip (bit n): query n did not select the block; all its keys are masked
//    (p = 0 through a reference of +inf in the exponent, max -inf).
//  * k0: the first half's K operands, from load_k_half on the same stage.
//  * hook(i) lets the caller place its own memory traffic in the block:
//    i = 0..3 at the start of the d-steps of S1, i = 4 right after them (Q is
//    no longer read from there on), i = 5..12 at the start of the PV regions.
//  * PRIO: the wave's issue priority over the block (s_setprio; the other
//    wave of the SIMD takes the issue slots it leaves): kPrioNone keeps it,
//    kPrioScores raises it through S0 .. [S1 | exp 0] and lowers it for the
//    second half, kPrioPv raises it through the P.V regions.
constexpr int kPrioNone = 0, kPrioScores = 1, kPrioPv = 2;
template <bool FIRST, bool MASKED, int VOFF = kVOff, int PRIO = kPrioNone, class QG, class H>
__device__ __forceinline__ void attend_block(QG& qg, const lds_char* stage_in, const KHalf& k0, const int* lim,
                                             float scale_log2, unsigned skip, H hook) {
  constexpr int QN = QG::kQN;
  constexpr int kExpValu = 21;  // VALU instructions of one exp_unit
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  // An opaque copy of the stage pointer keeps the operand reads next to their
  // MFMAs (otherwise they are hoisted across queries into many registers).
  const lds_char* stage = stage_in;
  asm volatile("" : "+v"(stage));
  f32x4 s0[QN][4], s1[QN][4];
  bf16x8 p0[QN][2], p1[QN][2];
  float mx[QN], mc[QN];

  if constexpr (PRIO == kPrioScores) __builtin_amdgcn_s_setprio(1);
  qk_half0(s0, qg.qop, k0, stage);
  // operands of the first pipelined step, read before the max and the branch
  bf16x8 ka[4], va[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) ka[t] = lds_k(stage, 4 + t, 0, c, qd);
  half_max<MASKED>(s0, lim, 0, mx);
#pragma unroll
  for (int n = 0; n < QN; ++n)
    if ((skip >> n) & 1u) mx[n] = -__builtin_inff();
  if (FIRST) {
#pragma unroll
    for (int n = 0; n < QN; ++n) qg.m[n] = mx[n];
  } else {
    bool need = false;
#pragma unroll
    for (int n = 0; n < QN; ++n) need |= (mx[n] - qg.m[n]) * scale_log2 > kLazy;
    if (__any(need)) {
#pragma unroll
      for (int n = 0; n < QN; ++n) {
        // alpha = 1 where the reference stays (also for m = mx = -inf)
        const float mnew = fmaxf(qg.m[n], mx[n]);
        const float alpha = mnew == qg.m[n] ? 1.0f : __builtin_amdgcn_exp2f((qg.m[n] - mnew) * scale_log2);
#pragma unroll
        for (int t = 0; t < 9; ++t) qg.o[n][t] *= alpha;
        qg.m[n] = mnew;
      }
    }
  }

  // S1 | exp 0
  {
#pragma unroll
    for (int n = 0; n < QN; ++n) {
      mc[n] = ((skip >> n) & 1u) ? __builtin_inff() : qg.m[n] * scale_log2;
#pragma unroll
      for (int t = 0; t < 4; ++t) s1[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 kn[4];
    static_for<0, 4>([&](auto ist) {
      constexpr int st = decltype(ist)::value;
      hook(st);
      if constexpr (st < 3) {
#pragma unroll
        for (int t = 0; t < 4; ++t) kn[t] = lds_k(stage, 4 + t, st + 1, c, qd);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int n = 0; n < QN; ++n) s1[n][t] = mfma16x16x32(ka[t], qg.qop[n][st], s1[n][t]);
      // exp units (n, j) = (u / 2, u % 2) of this step
      constexpr int u0 = (st * 2 * QN + 3) / 4, u1 = ((st + 1) * 2 * QN + 3) / 4;
#pragma unroll
      for (int u = u0; u < u1; ++u) exp_unit(s0, mc, scale_log2, p0, u >> 1, u & 1);
      sched_region<4 * QN, (u1 - u0) * kExpValu, st < 3 ? 4 : 0>();
#pragma unroll
      for (int t = 0; t < 4; ++t) ka[t] = kn[t];
    });
  }
  hook(4);
  if constexpr (PRIO == kPrioScores) __builtin_amdgcn_s_setprio(0);
  half_max<MASKED>(s1, lim, 1, mx);
#pragma unroll
  for (int n = 0; n < QN; ++n)
    if ((skip >> n) & 1u) mx[n] = -__builtin_inff();
  {
    bool need = false;
#pragma unroll
    for (int n = 0; n < QN; ++n) need |= (mx[n] - qg.m[n]) * scale_log2 > kLazy;
    if (__any(need)) {
      float alpha[QN];
#pragma unroll
      for (int n = 0; n < QN; ++n) {
        const float mnew = fmaxf(qg.m[n], mx[n]);
        alpha[n] = mnew == qg.m[n] ? 1.0f : __builtin_amdgcn_exp2f((qg.m[n] - mnew) * scale_log2);
        if (!FIRST) {
#pragma unroll
          for (int t = 0; t < 9; ++t) qg.o[n][t] *= alpha[n];
        }
        qg.m[n] = mnew;
      }
      scale_p(p0, alpha);
    }
  }

  // PV0 | exp 1, then PV1; each key step reads the next step's V^T operands
  {
    const uint32_t one2 = 0x3f803f80u;  // two bf16 ones
    const bf16x8 ones = as_bf16x8((u32x4){one2, one2, one2, one2});
#pragma unroll
    for (int n = 0; n < QN; ++n) mc[n] = ((skip >> n) & 1u) ? __builtin_inff() : qg.m[n] * scale_log2;
    // region r = 2*st + hh covers d-tiles 4hh .. 4hh+3 (+ the ones tile) of
    // key step st and reads the next region's V^T operands
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) va[dt] = lds_vt<VOFF>(stage, dt, 0, c, qd);
    if constexpr (PRIO == kPrioPv) __builtin_amdgcn_s_setprio(1);
    static_for<0, 8>([&](auto ir) {
      constexpr int r = decltype(ir)::value, st = r >> 1, hh = r & 1;
      constexpr int nst = hh ? st + 1 : st, nd0 = hh ? 0 : 4;
      hook(5 + r);
      if constexpr (nst < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) va[nd0 + i] = lds_vt<VOFF>(stage, nd0 + i, nst, c, qd);
      }
      constexpr int d0 = 4 * hh, d1 = hh ? 9 : 4;
#pragma unroll
      for (int dt = d0; dt < d1; ++dt) {
        const bf16x8 a = dt < 8 ? va[dt] : ones;
#pragma unroll
        for (int n = 0; n < QN; ++n) {
          const bf16x8 b = st < 2 ? p0[n][st & 1] : p1[n][st & 1];
          qg.o[n][dt] = (FIRST && st == 0) ? mfma16x16x32(a, b, (f32x4){0.f, 0.f, 0.f, 0.f})
                                           : mfma16x16x32(a, b, qg.o[n][dt]);
        }
      }
      // exp units of half 1 in the first four regions (PV0)
      constexpr int u0 = r < 4 ? (r * 2 * QN + 3) / 4 : 0, u1 = r < 4 ? ((r + 1) * 2 * QN + 3) / 4 : 0;
#pragma unroll
      for (int u = u0; u < u1; ++u) exp_unit(s1, mc, scale_log2, p1, u >> 1, u & 1);
      sched_region<(d1 - d0) * QN, (u1 - u0) * kExpValu, nst < 4 ? 8 : 0>();
    });
    if constexpr (PRIO == kPrioPv) __builtin_amdgcn_s_setprio(0);
  }
}

// Online-softmax update with one staged block of NT key tiles (NT = BK/16 =
// 2 or 4: a block of 32 or 64 keys in the first rows of the stage): the
// arithmetic of attend_block (scores kept raw, lazy rescale, the denominator
// accumulated through a tile of ones) on the block's keys only, without the
// two-half pipelining. MASKED, skip and hook as in attend_block (hook(4) once
// Q is no longer read).
template <bool FIRST, bool MASKED, int NT, int VOFF = kVOff, class QG, class H>
__device__ __forceinline__ void attend_short(QG& qg, const lds_char* stage, const int* lim, float scale_log2,
                                             unsigned skip, H hook) {
  static_assert(NT == 2 || NT == 4, "blocks of 32 or 64 keys");
  constexpr int QN = QG::kQN;
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  f32x4 s[QN][4];
#pragma unroll
  for (int n = 0; n < QN; ++n)
#pragma unroll
    for (int t = 0; t < 4; ++t) s[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    hook(st);
    bf16x8 a[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) a[t] = lds_k(stage, t, st, c, qd);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int n = 0; n < QN; ++n) s[n][t] = mfma16x16x32(a[t], qg.qop[n][st], s[n][t]);
  }
  hook(4);
  float mx[QN], mc[QN];
#pragma unroll
  for (int n = 0; n < QN; ++n) {
    if (MASKED) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * t + 4 * qd + r > lim[n]) s[n][t][r] = -__builtin_inff();
    }
    float x = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < NT; ++t) x = fmaxf(fmaxf(x, fmaxf(s[n][t][0], s[n][t][1])), fmaxf(s[n][t][2], s[n][t][3]));
    mx[n] = ((skip >> n) & 1u) ? -__builtin_inff() : max_lane_groups(x);
  }
  if (FIRST) {
#pragma unroll
    for (int n = 0; n < QN; ++n) qg.m[n] = mx[n];
  } else {
    bool need = false;
#pragma unroll
    for (int n = 0; n < QN; ++n) need |= (mx[n] - qg.m[n]) * scale_log2 > kLazy;
    if (__any(need)) {
#pragma unroll
      for (int n = 0; n < QN; ++n) {
        const float mnew = fmaxf(qg.m[n], mx[n]);
        const float alpha = mnew == qg.m[n] ? 1.0f : __builtin_amdgcn_exp2f((qg.m[n] - mnew) * scale_log2);
#pragma unroll
        for (int t = 0; t < 9; ++t) qg.o[n][t] *= alpha;
        qg.m[n] = mnew;
      }
    }
  }
  bf16x8 p[QN][2];
#pragma unroll
  for (int n = 0; n < QN; ++n) {
    mc[n] = ((skip >> n) & 1u) ? __builtin_inff() : qg.m[n] * scale_log2;
#pragma unroll
    for (int j = 0; j < NT / 2; ++j) exp_unit(s, mc, scale_log2, p, n, j);
  }
  const uint32_t one2 = 0x3f803f80u;  // two bf16 ones
  const bf16x8 ones = as_bf16x8((u32x4){one2, one2, one2, one2});
#pragma unroll
  for (int st = 0; st < NT / 2; ++st) {
    hook(5 + st);
    bf16x8 va[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = lds_vt<VOFF>(stage, dt, st, c, qd);
#pragma unroll
    for (int dt = 0; dt < 9; ++dt) {
      const bf16x8 a = dt < 8 ? va[dt] : ones;
#pragma unroll
      for (int n = 0; n < QN; ++n)
        qg.o[n][dt] = (FIRST && st == 0) ? mfma16x16x32(a, p[n][st], (f32x4){0.f, 0.f, 0.f, 0.f})
                                         : mfma16x16x32(a, p[n][st], qg.o[n][dt]);
    }
  }
#pragma unroll
  for (int i = 5 + NT / 2; i < 13; ++i) hook(i);
}

// Softmax partial of one query, normalised, in fragment order: element (head
// c, dim 16dt + 4qd + r) sits at dt*256 + (16qd + c)*4 + r of the 2048-element
// slot, so each of the eight stores of a wave writes 512 contiguous bytes.
// lse2 = m*c + log2(l) per head (c = scale * log2 e). It issues
// kStorePartialOps vector memory instructions: the 8 fragment stores (512 B
// apart per lane, never merged) and the lse store.
constexpr int kStorePartialOps = 9;
__device__ __forceinline__ void store_partial(const f32x4 (&o)[9], float m, float scale_log2, uint16_t* dst,
                                              float* lse16) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  const float l = o[8][0];
  const float inv = 1.0f / l;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
    *reinterpret_cast<u32x2*>(dst + dt * 256 + lane * 4) = w;
  }
  if (qd == 0) lse16[c] = m * scale_log2 + __builtin_amdgcn_logf(l);
}

// Issue the direct-to-LDS loads of one partial (4 KiB, copied as is) into
// `dst`: four loads per wave.
__device__ __forceinline__ void stage_partial(const uint16_t* src, lds_char* dst) {
  const uint32_t voff = (threadIdx.x & 63) * 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) lds_dma16_s(src + j * 512, voff, dst + j * 1024);
}

// MFMA 16x16x16 bf16: lane (i, g) holds A[i][4g + j] and B[4g + j][i] (j < 4);
// the result layout is that of the 16x16x32 product.
__device__ __forceinline__ f32x4 mfma16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// A operand of the merge MFMA for d-tile dt of a staged partial X: lane (c,
// qd) holds X[4qd + j][16dt + c] at k = 4qd + j, read transposed: lane i of a
// 16-lane group addresses head 4qd + i/4, dims 16dt + 4(i%4) .. +3, the 8-byte
// piece at dt*512 + (16(i%4) + head)*8 of the fragment-order slot.
__device__ __forceinline__ i16x4 partial_operand(const lds_char* xs, int dt, int c, int qd) {
  const int r = 4 * qd + (c >> 2);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(xs + dt * 512 + (16 * (c & 3) + r) * 8));
}

// B operand diag(x) paired with partial_operand: row k = 4qd + j of column
// (head) c is x at k == c, else 0; `bits` is x as bf16.
__device__ __forceinline__ i16x4 diag_operand(uint32_t bits, int c, int qd) {
  const uint32_t h = qd == (c >> 2) ? bits << ((c & 1) * 16) : 0u;
  const bool odd = (c & 2) != 0;
  return __builtin_bit_cast(i16x4, (u32x2){odd ? 0u : h, odd ? h : 0u});
}

// Merge of a normalised partial (staged at xs, lse2 lp for the lane's head)
// into query n's running state (o, l = o[8], reference max m): o += w X^T and
// l += w with w = 2^(lp - m*c), as MFMAs against diag(w_hi) and diag(w_lo),
// the bf16 rounding of w and of its remainder (w to about 16 bits; the ones
// tile adds w to l), after a lazy rescale of the state when lp exceeds m*c by
// more than kLazy (a fresh state, m = -inf, takes m*c = lp).
template <int N, class QG>
__device__ __forceinline__ void merge_partial(QG& qg, const lds_char* xs, float lp, float scale_log2) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  i16x4 a[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) a[dt] = partial_operand(xs, dt, c, qd);
  float mc = qg.m[N] * scale_log2;
  if (__any(lp - mc > kLazy)) {
    const float mnew = fmaxf(mc, lp);
    const float alpha = __builtin_amdgcn_exp2f(mc - mnew);
#pragma unroll
    for (int t = 0; t < 9; ++t) qg.o[N][t] *= alpha;
    qg.m[N] = mnew / scale_log2;
    mc = mnew;
  }
  const float w = __builtin_amdgcn_exp2f(lp - mc);
  const uint32_t hi = pack_bf16x2(w, 0.f) & 0xffffu;
  const uint32_t lo = pack_bf16x2(w - bf2f(hi), 0.f) & 0xffffu;
  const i16x4 bh = diag_operand(hi, c, qd), bl = diag_operand(lo, c, qd);
  const uint32_t one2 = 0x3f803f80u;
  const i16x4 ones = __builtin_bit_cast(i16x4, (u32x2){one2, one2});
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) qg.o[N][dt] = mfma16x16x16(a[dt], bh, qg.o[N][dt]);
  qg.o[N][8] = mfma16x16x16(ones, bh, qg.o[N][8]);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) qg.o[N][dt] = mfma16x16x16(a[dt], bl, qg.o[N][dt]);
  qg.o[N][8] = mfma16x16x16(ones, bl, qg.o[N][8]);
}

// merge_partial into query pn (wave-uniform) of the group.
template <class QG>
__device__ __forceinline__ void merge_partial_into(QG& qg, int pn, const lds_char* xs, float lp, float scale_log2) {
  static_for<0, QG::kQN>([&](auto in) {
    constexpr int n = decltype(in)::value;
    if (pn == n) merge_partial<n>(qg, xs, lp, scale_log2);
  });
}

constexpr int kAttnQN = 2;
constexpr int kAttnWaves = 8;

// Sparse (KV-outer) part: one persistent workgroup per CU drains the tile
// queue. A query's own block is always shared by its whole 16-row unit, so no
// KV-outer tile needs causal masking. A tile holds at most 16 queries; wave w
// takes its entries 2w and 2w+1. Everything a tile needs is fetched one tile
// ahead, so no latency sits between two tiles: while tile j is computed, the
// K/V of tile j+1 stream into the other LDS stage, the wave's entries of tile
// j+1 and then their Q are loaded, and the descriptor of tile j+2 is read.
// Tiles are claimed from the queue kClaim at a time, one chunk ahead. Each
// wave raises its issue priority through the scores of a block
// (kPrioScores): its waves drift apart between tiles, and the other wave of
// the SIMD fills the slots left meanwhile.
template <int BK>
__global__ __launch_bounds__(512, 1) void k_attn_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ tiles, int32_t* __restrict__ tile_info,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, int64_t n_tokens, int G,
    int nbw, int topk, float scale_log2, int32_t* __restrict__ tile_visits, int64_t* __restrict__ wg_trace) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage];
  __shared__ int s_t[4];
  lds_char* lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, qd = lane >> 4;
  const int T = tile_info[0];
  const int Hq = G * kHpg;
  const int64_t rstride = (int64_t)G * kHeadDim;
  const int e0 = wave * kAttnQN;  // the wave's entries in every tile

  const StageOffsets soff = stage_offsets(rstride, wave);
  struct Tile {
    int t, begin, len, g, b;
  };
  auto read_tile = [&](int t) -> Tile {
    Tile d{t, 0, 0, 0, 0};
    if (t < T) {
      d.g = tiles[4 * t];
      d.begin = tiles[4 * t + 1];
      d.len = tiles[4 * t + 2];
      d.b = tiles[4 * t + 3];
    }
    return d;
  };
  auto stage_tile = [&](const Tile& d, lds_char* dst) {
    const uint64_t e = block_elems(d.b, BK, G, d.g);
    stage_block_bk<BK>(dst, k + e, v + e, rstride, (int)min<int64_t>(BK, n_tokens - (int64_t)d.b * BK), wave,
                       kAttnWaves, soff);
  };
  QueryGroup<kAttnQN> qg;
  auto fetch_q = [&](const int (&ent)[kAttnQN], int tg) {
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) {
      const int64_t i_rel = ent[n] >> 4;
      load_q(qg, n, q + ((i_rel * Hq) + tg * kHpg + c) * kHeadDim + 8 * qd);
    }
  };
  auto read_entries = [&](const Tile& d, int (&ent)[kAttnQN]) {
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) ent[n] = entries[d.begin + min(e0 + n, d.len - 1)];
  };

  // the queue: chunk c of this workgroup's tiles (tiles kClaim*c ..) starts at
  // queue position s_t[c & 1]
  constexpr int kClaim = kTileClaim;
  // chunk c+1 is claimed at tile kClaim*c and first read for tile kClaim*c + 2
  // (the descriptor two tiles ahead): a barrier lies between only if the
  // chunk is longer than two tiles
  static_assert(kClaim >= 3, "the claim must be visible before the look-ahead reads it");
  const int64_t t_start = wall_clock64();
  if (tid == 0) {
    if (blockIdx.x == 0) tile_info[4] = gridDim.x;
    s_t[0] = atomicAdd(&tile_info[1], kClaim);
  }
  __syncthreads();
  auto tile_pos = [&](int jj) { return __builtin_amdgcn_readfirstlane(s_t[(jj / kClaim) & 1] + jj % kClaim); };
  Tile cur = read_tile(tile_pos(0));
  Tile nxt = read_tile(tile_pos(1));
  int ent[kAttnQN] = {0, 0};
  if (cur.t < T) {
    stage_tile(cur, lds);
    if (e0 < cur.len) {
      read_entries(cur, ent);
      fetch_q(ent, cur.g);
    }
  }
  // vector memory operations issued after the last stage load, counted from
  // the operations they certainly are (an over-count would let the wait pass
  // with stage loads still in flight)
  int after_dma = 0;
  int drained = 0;    // tiles this workgroup computed
  for (int j = 0; cur.t < T; ++j) {
    wait_vmcnt_upto(after_dma);  // the stage of tile j is in
    wait_lgkmcnt0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // ... for every wave; the other stage is free; s_t visible
    asm volatile("" ::: "memory");
    const lds_char* stage = lds + (j & 1) * kStage;
    KHalf k0;
    if (BK == kBlock && e0 < cur.len) load_k_half(k0, stage);
    // chunk c+1 is claimed when chunk c starts; it is first read two tiles
    // later (for tile kClaim*(c+1)), after at least one more barrier. Both
    // atomics are issued before the next stage's loads, so the vmcnt budget
    // of those loads (after_dma) does not count them.
    if (tid == 0) {
      atomicAdd(&tile_visits[cur.t], 1);
      if (j % kClaim == 0) s_t[(j / kClaim + 1) & 1] = atomicAdd(&tile_info[1], kClaim);
    }
    const int t2 = tile_pos(j + 2);
    int d2[4] = {0, 0, 0, 0};
    if (t2 < T) {
      d2[0] = tiles[4 * t2];
      d2[1] = tiles[4 * t2 + 1];
      d2[2] = tiles[4 * t2 + 2];
      d2[3] = tiles[4 * t2 + 3];
    }
    after_dma = 0;
    if (nxt.t < T) stage_tile(nxt, lds + ((j + 1) & 1) * kStage);
    const bool next_work = nxt.t < T && e0 < nxt.len;
    int nent[kAttnQN] = {0, 0};
    if (next_work) {
      read_entries(nxt, nent);
      // their Q, below (the entries are not counted: their address is
      // wave-uniform, so they may be scalar loads, which vmcnt does not
      // track; left out, a vector load only makes the wait stronger)
      after_dma += kAttnQN * kLoadQOps;
    }
    if (e0 < cur.len) {
      // once the scores no longer need Q, the next tile's is loaded
      auto hook = [&](int i) {
        if (i == 4 && next_work) fetch_q(nent, nxt.g);
      };
      if constexpr (BK == kBlock)
        attend_block<true, false, kVOff, kPrioScores>(qg, stage, k0, nullptr, scale_log2, 0u, hook);
      else
        attend_short<true, false, BK / 16>(qg, stage, nullptr, scale_log2, 0u, hook);
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) {
        if (e0 + n < cur.len) {
          const int64_t slot = ((int64_t)(ent[n] >> 4) * G + cur.g) * topk + (ent[n] & 15);
          store_partial(qg.o[n], qg.m[n], scale_log2, part_o + slot * kHpg * kHeadDim, part_lse + slot * kHpg);
          after_dma += kStorePartialOps;
        }
      }
    } else if (next_work) {
      fetch_q(nent, nxt.g);
    }
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) ent[n] = nent[n];
    cur = nxt;
    nxt.t = t2;
    nxt.begin = d2[1];
    nxt.len = d2[2];
    nxt.g = d2[0];
    nxt.b = d2[3];
    if (tid == 0) ++drained;
  }
  if (tid == 0) {
    int64_t* r = wg_trace + 4 * blockIdx.x;
    r[0] = __smid();
    r[1] = drained;
    r[2] = t_start;
    r[3] = wall_clock64();
  }
}

// Dense part and final merge: blocks selected by at least kDenseMin rows of a
// 16-query unit (by all of them, if the unit has fewer) are computed
// query-stationary (FlashAttention-style online softmax over the unit's list;
// each block is staged once for all 16 queries, the next one streaming into
// the other stage meanwhile). Rows that did not select a listed block are
// masked for it; a wave whose two rows both did not skips it. Eight waves per
// (unit, group) item, two queries per wave. The list always ends with
// the unit's own block, the only one that needs the causal mask. This pass
// runs after the KV-outer pass and merges its partials (the slots of the
// query's selection outside the unit's list) into the same online state, so
// every row's output and lse are written here, once, without atomics (the
// second phase of the two-phase combine [pnsm, section 7]):
//   out = o / l,   lse = (m*c + log2 l) * ln 2.
// The grid is persistent (one workgroup per CU) and the (group, unit) items
// are split into kXcd contiguous ranges, one per XCD, each drained through a
// counter of its own (tile_info[8 + x], zeroed with the tile queue;
// tile_info[7] gets the grid size): units that share K/V blocks then meet in
// one L2. The next unit is claimed when a unit starts; its list, row masks,
// count and slots stream into LDS during the unit's last block, its Q loads
// while the unit's output is stored, and its first block is staged right
// after. A workgroup whose range is drained takes items from the other
// ranges in turn.
template <int BK>
__global__ __launch_bounds__(512, 1) void k_attn_dense(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ dense_cnt, const int32_t* __restrict__ dense_list,
    const int32_t* __restrict__ dense_qmask, const int32_t* __restrict__ dense_slots, const uint16_t* __restrict__ part_o,
    const float* __restrict__ part_lse, uint16_t* __restrict__ out, float* __restrict__ lse_out, int64_t n_tokens,
    int64_t row0, int nrows, int nunits, int G, int topk, float scale_log2,
    int32_t* __restrict__ tile_info) {
  // two K/V stages, 256 bytes per wave for the partials' lse, then the next
  // unit's metadata (768 bytes + 256 per wave)
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage + kAttnWaves * 256 + 768 + kAttnWaves * 256];
  __shared__ int s_next[2];
  lds_char* lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, qd = lane >> 4;
  const int Hq = G * kHpg;
  const int64_t rstride = (int64_t)G * kHeadDim;
  const StageOffsets soff = stage_offsets(rstride, wave);
  // items (group, unit) in group-major order, split into kXcd ranges; range
  // r is [r*q + min(r, rm), + q + (r < rm)). XCD x = blockIdx.x mod kXcd (the
  // dispatcher's order: only the locality depends on it) drains range x
  // first, then the others (victim: the range it currently takes from).
  // Claims are made by thread 0.
  const int nitems = nunits * G;
  const int iq = nitems / kXcd, rm = nitems % kXcd;
  int victim = blockIdx.x % kXcd;
  auto claim_from = [&](int r) -> int {
    const int t = atomicAdd(tile_info + 8 + r, 1);
    return t < iq + (r < rm ? 1 : 0) ? r * iq + min(r, rm) + t : -1;
  };
  // (waits for each claim: used where the result is needed at once)
  auto claim_any = [&]() -> int {
    for (int t = 0; t < kXcd; ++t) {
      const int it = claim_from(victim);
      if (it >= 0) return it;
      victim = victim + 1 < kXcd ? victim + 1 : 0;
    }
    return -1;
  };

  // a unit's list and the rows that selected each entry (lane j holds entry
  // j, read back with a uniform readlane; entries past the count are not
  // used), its count and its rows' dense slots; then the queries' Q
  int lane_blk = 0, lane_qm = 0, nd = 0;
  int slots[kAttnQN];
  QueryGroup<kAttnQN> qg;
  auto unit_loads = [&](int it) {
    const int ug = it / nunits, uu = it - ug * nunits;
    const int64_t l0 = ((int64_t)ug * nunits + uu) * kDenseMax;
    lane_blk = dense_list[l0 + lane];
    lane_qm = dense_qmask[l0 + lane];
    nd = dense_cnt[ug * nunits + uu];  // >= 1: the unit's own block
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n)
      slots[n] = dense_slots[(int64_t)ug * nrows + min(uu * 16 + wave * kAttnQN + n, nrows - 1)];
  };
  auto unit_q = [&](int it) {
    const int ug = it / nunits, uu = it - ug * nunits;
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) {
      const int64_t i_rel = min(uu * 16 + wave * kAttnQN + n, nrows - 1);
      load_q(qg, n, q + ((i_rel * Hq) + ug * kHpg + c) * kHeadDim + 8 * qd);
    }
  };
  // The same metadata of the next unit copied into LDS (meta: list, row
  // masks, count, then 256 bytes of slots per wave), so that no registers hold
  // it during the current unit's last block and merges, and read back.
  lds_char* meta = lds + 2 * kStage + kAttnWaves * 256;
  auto meta_loads = [&](int it) {
    const int ug = it / nunits, uu = it - ug * nunits;
    const int64_t l0 = ((int64_t)ug * nunits + uu) * kDenseMax;
    if (wave == 0) lds_dma4(dense_list + l0 + lane, meta);
    if (wave == 1) lds_dma4(dense_qmask + l0 + lane, meta + 256);
    if (wave == 2) lds_dma4(dense_cnt + ug * nunits + uu, meta + 512);
    lds_dma4(dense_slots + (int64_t)ug * nrows + min(uu * 16 + wave * kAttnQN + (lane & 1), nrows - 1),
             meta + 768 + wave * 256);
  };
  auto meta_read = [&]() {
    typedef __attribute__((address_space(3))) const int lds_int;
    lane_blk = ((lds_int*)meta)[lane];
    lane_qm = ((lds_int*)(meta + 256))[lane];
    nd = __builtin_amdgcn_readfirstlane(((lds_int*)(meta + 512))[0]);
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) slots[n] = ((lds_int*)(meta + 768 + wave * 256))[n];
  };
  // the unit's first block into stage 0 (every wave)
  auto stage_first = [&](int it) {
    const int ug = it / nunits;
    const int b0 = __builtin_amdgcn_readfirstlane(lane_blk);
    const uint64_t e = block_elems(b0, BK, G, ug);
    stage_block_bk<BK>(lds, k + e, v + e, rstride, (int)min<int64_t>(BK, n_tokens - (int64_t)b0 * BK), wave,
                       kAttnWaves, soff);
  };

  if (tid == 0) {
    if (blockIdx.x == 0) tile_info[7] = gridDim.x;
    s_next[0] = claim_any();
  }
  __syncthreads();
  int item = s_next[0];
  if (item < 0) return;
  unit_loads(item);
  unit_q(item);
  stage_first(item);
  for (int par = 1;; par ^= 1) {
    const int g = item / nunits, unit = item - g * nunits;
    const int i_rel0 = unit * 16 + wave * kAttnQN;
    const int b_loc = (int)((row0 + unit * 16) / BK);
    const int nsel = min(topk, b_loc + 1);
    // the next item from the current range, claimed now and waited for only
    // where it is published
    int claimed = -1;
    if (tid == 0) claimed = claim_from(victim);
    // slots of each query's selection computed KV-outer: the valid ones the
    // dense pass does not cover
    uint32_t use[kAttnQN];
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n)
      use[n] = i_rel0 + n < nrows ? (uint32_t)__builtin_amdgcn_readfirstlane(~slots[n]) & ((1u << nsel) - 1u) : 0u;
    reset_state(qg);

    // KV-outer partials of the wave's queries, in (query, slot) order, merged
    // after the last block (below). Merging them between blocks instead costs
    // more: the waves' partial counts differ, and every block's barrier then
    // waits for the wave with the most.
    lds_char* lse_side = lds + 2 * kStage + wave * 256;  // [region][partial][16 heads] fp32
    // (wave-uniform bookkeeping, kept in scalar registers; slot indices fit 32
    // bits: rows * G * topk of a window)
    int cur_n = 0;
    uint32_t cur_rem = use[0];
    auto next_pair = [&](int& pn, int64_t& slot) -> bool {
#pragma unroll
      for (int n = 1; n < kAttnQN; ++n)
        if (cur_rem == 0u && cur_n == n - 1) {
          cur_n = n;
          cur_rem = use[n];
        }
      if (cur_rem == 0u) return false;
      const int pu = __builtin_ctz(cur_rem);
      cur_rem &= cur_rem - 1u;
      pn = cur_n;
      slot = (uint32_t)__builtin_amdgcn_readfirstlane(((i_rel0 + cur_n) * G + g) * topk + pu);
      return true;
    };

    // shared older blocks (unmasked), then the unit's own block (masked)
    for (int d = 0; d + 1 < nd; ++d) {
      wait_loads();
      __syncthreads();  // stage d&1 complete; stage (d+1)&1 free
      KHalf k0;
      if constexpr (BK == kBlock) load_k_half(k0, lds + (d & 1) * kStage);
      // block d+1 streams into the other stage, loaded by waves 0-3 only (one
      // per SIMD): their partners start computing while they wait for room in
      // the memory queue
      const int b2 = __builtin_amdgcn_readlane(lane_blk, d + 1);
      const uint64_t e2 = block_elems(b2, BK, G, g);
      if (wave < 4)
        stage_block_bk<BK>(lds + ((d + 1) & 1) * kStage, k + e2, v + e2, rstride,
                           (int)min<int64_t>(BK, n_tokens - (int64_t)b2 * BK), wave, 4, soff);
      // queries of the wave that did not select the block are masked; a wave
      // with none that did skips it
      const unsigned skip =
          ~((unsigned)__builtin_amdgcn_readlane(lane_qm, d) >> (wave * kAttnQN)) & ((1u << kAttnQN) - 1u);
      if (skip != (1u << kAttnQN) - 1u) {
        if constexpr (BK == kBlock)
          attend_block<false, false>(qg, lds + (d & 1) * kStage, k0, nullptr, scale_log2, skip, [](int) {});
        else
          attend_short<false, false, BK / 16>(qg, lds + (d & 1) * kStage, nullptr, scale_log2, skip, [](int) {});
      }
    }

    // The partials stream through two 8 KiB LDS regions of the wave (two
    // partials each, direct-to-LDS loads, their lse into the wave's lse_side):
    // region 0 in the stage not holding the last block, filled while the last
    // block is computed; region 1 in the last block's stage once every wave is
    // done with it. Completion is tracked with vmcnt (5 loads per partial), so
    // one region is merged while the other streams in.
    const int last = (nd - 1) & 1;
    lds_char* region[2] = {lds + (last ^ 1) * kStage + wave * 8192, lds + last * kStage + wave * 8192};
    auto issue_round = [&](int reg, int& cnt, int& na, int& nb) {
      cnt = 0;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        int pn = 0;
        int64_t slot = 0;
        if (!next_pair(pn, slot)) break;
        stage_partial(part_o + slot * (kHpg * kHeadDim), region[reg] + p * 4096);
        if (lane < kHpg) lds_dma4(part_lse + slot * kHpg + lane, lse_side + reg * 128 + p * 64);
        if (p == 0) na = pn; else nb = pn;
        cnt = p + 1;
      }
    };
    auto wait_round = [](int cnt_in_flight) {
      if (cnt_in_flight == 2)
        wait_vmcnt10();
      else if (cnt_in_flight == 1)
        wait_vmcnt5();
      else
        wait_vmcnt0();
    };
    auto merge_round = [&](int reg, int cnt, int na, int nb) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (p >= cnt) break;
        const float lp = *(const __attribute__((address_space(3))) float*)(lse_side + reg * 128 + p * 64 + c * 4);
        merge_partial_into(qg, p ? nb : na, region[reg] + p * 4096, lp, scale_log2);
      }
      wait_lgkmcnt0();  // region read out before it is refilled
    };
    int cA = 0, nA0 = 0, nA1 = 0, cB = 0, nB0 = 0, nB1 = 0;
    // the next item (waiting for the claims only once this range is drained)
    if (tid == 0) s_next[par] = claimed >= 0 ? claimed : claim_any();
    int next;
    {
      wait_loads();
      __syncthreads();  // (also publishes s_next[par])
      next = s_next[par];
      // the next unit's list, row masks, count and slots stream into LDS
      // while this unit's last block is computed
      if (next >= 0) meta_loads(next);
      KHalf k0;
      if constexpr (BK == kBlock) load_k_half(k0, lds + last * kStage);
      issue_round(0, cA, nA0, nA1);
      int lim[kAttnQN];
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) lim[n] = (int)(min(i_rel0 + n, nrows - 1) + row0 - (int64_t)b_loc * BK);
      if constexpr (BK == kBlock)
        attend_block<false, true>(qg, lds + last * kStage, k0, lim, scale_log2, 0u, [](int) {});
      else
        attend_short<false, true, BK / 16>(qg, lds + last * kStage, lim, scale_log2, 0u, [](int) {});
    }
    wait_lgkmcnt0();  // the last block's stage is free
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_round(1, cB, nB0, nB1);
    // rounds alternate regions; pairs are handed out in order, so an empty
    // round means every later round is empty too
    while (cA > 0) {
      wait_round(cB);
      merge_round(0, cA, nA0, nA1);
      issue_round(0, cA, nA0, nA1);
      if (cB == 0) break;
      wait_round(cA);
      merge_round(1, cB, nB0, nB1);
      issue_round(1, cB, nB0, nB1);
    }
    // every wave is done with both stages before the next unit's first block
    // is staged (after the stores below), and every wave's copies of the next
    // unit's metadata have landed; its Q loads meanwhile
    wait_vmcnt0();
    lds_barrier();
    if (next >= 0) {
      meta_read();
      unit_q(next);
    }
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) {
      const int i_rel = i_rel0 + n;
      if (i_rel >= nrows) continue;
      const float l = qg.o[n][8][0];
      const float inv = 1.0f / l;
      uint16_t* dst = out + ((int64_t)i_rel * Hq + g * kHpg + c) * kHeadDim + 4 * qd;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        u32x2 w = {pack_bf16x2(qg.o[n][dt][0] * inv, qg.o[n][dt][1] * inv),
                   pack_bf16x2(qg.o[n][dt][2] * inv, qg.o[n][dt][3] * inv)};
        *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
      }
      if (lse_out && qd == 0)
        lse_out[(int64_t)i_rel * Hq + g * kHpg + c] =
            (qg.m[n] * scale_log2 + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
    }
    if (next < 0) break;
    stage_first(next);
    item = next;
  }
}

// Decode: one workgroup per (sequence, group). It first selects its row's
// blocks from the pooled index scores (the own block plus the k-1 best older
// ones, ranked by its four waves; written to sel_out when given), then the
// selected blocks stream through two LDS stages (all four waves issue the
// direct-to-LDS loads of the next block while wave 0 computes the current
// one), and wave 0 keeps the group's 16 heads in one online-softmax state
// across the blocks (the own block, the last in ascending order, with the
// causal mask), so the output and lse are written at the end with no partials
// and no separate combine. Only cache rows below ctx_len are staged (later
// rows may hold anything).
constexpr int kDecWaves = 4;
template <int BK>
__global__ __launch_bounds__(kDecWaves * 64) void k_attn_decode(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, const float* __restrict__ sblk, int nb, int32_t* __restrict__ sel_out,
    uint16_t* __restrict__ out, float* __restrict__ lse_out, int64_t max_ctx, int G, int topk, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage];
  __shared__ float s_sv[kDecWaves * (kMaxTopk - 1)];
  __shared__ int s_si[kDecWaves * (kMaxTopk - 1)];
  __shared__ int s_cnt[2 * kDecWaves];
  __shared__ int s_tmp[kMaxTopk];
  __shared__ int s_ctr;
  __shared__ int s_sel[kMaxTopk];
  lds_char* lds = (lds_char*)lds_raw;
  const int item = blockIdx.x;  // sq * G + g
  const int sq = item / G, g = item % G;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c = lane & 15, qd = lane >> 4;
  const int64_t i = ctx_lens[sq] - 1;
  const int b_loc = (int)(i / BK);
  const int nsel = min(topk, b_loc + 1);
  const int Hq = G * kHpg;
  const int64_t rstride = (int64_t)G * kHeadDim;
  const int64_t seq0 = (int64_t)sq * max_ctx * G * kHeadDim + (int64_t)g * kHeadDim;
  // the selection: every block when there are at most k, else the k-1 best
  // older blocks (ascending) and the own block
  const StageOffsets soff = stage_offsets(rstride, wave);
  auto stage_blk = [&](int b, lds_char* dst) {
    const int64_t key0 = (int64_t)b * BK;
    const int64_t base = seq0 + key0 * rstride;
    stage_block_bk<BK>(dst, k + base, v + base, rstride, (int)min<int64_t>(BK, i + 1 - key0), wave, kDecWaves,
                       soff);
  };
  // the own block is known before the ranking: it is staged (and attended)
  // first, its loads issued once the ranking has read its candidates, so
  // they overlap the ranking
  auto stage_own = [&] { stage_blk(b_loc, lds); };
  QueryGroup<1> qg;
  if (wave == 0) {
    load_q(qg, 0, q + ((int64_t)sq * Hq + g * kHpg + c) * kHeadDim + 8 * qd);
    reset_state(qg);
  }
  if (b_loc < topk) {
    stage_own();
    if (wave == 0 && lane < topk) s_sel[lane] = lane <= b_loc ? lane : -1;
  } else {
    const float* row = sblk + (int64_t)item * nb;
    // up to 2048 candidates: a threshold search over the four waves (at 1024,
    // 9 us against 13 us for k-1 wave-wide pops; wave 0 alone took 19 us);
    // beyond, where the search's per-step barriers and counts cost more than
    // the pops, k-1 rounds over per-lane sorted lists
    if (b_loc <= 4 * 64 * kDecWaves)
      select_row_thr<kDecWaves, 4>(row, b_loc, topk - 1, s_cnt, s_tmp, &s_ctr, s_sel, stage_own);
    else if (b_loc <= 8 * 64 * kDecWaves)
      select_row_thr<kDecWaves, 8>(row, b_loc, topk - 1, s_cnt, s_tmp, &s_ctr, s_sel, stage_own);
    else
      select_row_rt<kDecWaves>(row, b_loc, topk - 1, s_sv, s_si, s_sel, stage_own);
    if (wave == 0 && lane == 0) s_sel[topk - 1] = b_loc;
  }
  lds_barrier();  // (the own block's loads stay in flight)
  // lane u holds slot u of the selection (ascending; the first nsel are valid,
  // the own block last)
  const int lane_blk = lane < topk ? s_sel[lane] : 0;
  if (sel_out && wave == 0 && lane < topk) sel_out[(int64_t)item * topk + lane] = lane_blk;
  // visit order: the own block, then the older blocks ascending
  auto block_at = [&](int u) { return u == 0 ? b_loc : __builtin_amdgcn_readlane(lane_blk, u - 1); };
  for (int u = 0; u < nsel; ++u) {
    wait_loads();
    __syncthreads();  // stage u&1 complete; stage (u+1)&1 free
    if (u + 1 < nsel) stage_blk(block_at(u + 1), lds + ((u + 1) & 1) * kStage);
    if (wave != 0) continue;
    const lds_char* st = lds + (u & 1) * kStage;
    if (u > 0) {  // an older block: every key is before the query
      if constexpr (BK == kBlock) {
        KHalf k0;
        load_k_half(k0, st);
        attend_block<false, false>(qg, st, k0, nullptr, scale_log2, 0u, [](int) {});
      } else {
        attend_short<false, false, BK / 16>(qg, st, nullptr, scale_log2, 0u, [](int) {});
      }
    } else {  // the own block, keys up to the query
      int lim[1] = {(int)(i - (int64_t)b_loc * BK)};
      if constexpr (BK == kBlock) {
        KHalf k0;
        load_k_half(k0, st);
        attend_block<false, true>(qg, st, k0, lim, scale_log2, 0u, [](int) {});
      } else {
        attend_short<false, true, BK / 16>(qg, st, lim, scale_log2, 0u, [](int) {});
      }
    }
  }
  if (wave != 0) return;
  const float l = qg.o[0][8][0];
  const float inv = 1.0f / l;
  uint16_t* dst = out + ((int64_t)sq * Hq + g * kHpg + c) * kHeadDim + 4 * qd;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w = {pack_bf16x2(qg.o[0][dt][0] * inv, qg.o[0][dt][1] * inv),
               pack_bf16x2(qg.o[0][dt][2] * inv, qg.o[0][dt][3] * inv)};
    *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
  }
  if (lse_out && qd == 0)
    lse_out[(int64_t)sq * Hq + g * kHpg + c] = (qg.m[0] * scale_log2 + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
}

template <int BK>
static void launch_attn_prefill_bk(const LaunchAttnPrefill& a, hipStream_t st) {
  hipLaunchKernelGGL(k_attn_prefill<BK>, dim3(a.grid), dim3(512), 0, st, a.q, a.k, a.v, a.entries, a.tiles,
                     a.tile_info, a.part_o, a.part_lse, a.n_tokens, a.G, a.nbw, a.topk, a.scale_log2,
                     a.tile_visits, a.wg_trace);
}

void launch_attn_prefill(const LaunchAttnPrefill& a, hipStream_t st) {
  switch (a.bk) {
    case 128: launch_attn_prefill_bk<128>(a, st); break;
    case 64: launch_attn_prefill_bk<64>(a, st); break;
    case 32: launch_attn_prefill_bk<32>(a, st); break;
    default: break;
  }
}

template <int BK>
static void launch_attn_dense_bk(const LaunchAttnDense& a, hipStream_t st) {
  hipLaunchKernelGGL(k_attn_dense<BK>, dim3(a.grid), dim3(kAttnWaves * 64), 0, st, a.q, a.k, a.v, a.dense_cnt,
                     a.dense_list, a.dense_qmask, a.dense_slots, a.part_o, a.part_lse, a.out, a.lse_out, a.n_tokens,
                     a.row0, a.nrows, a.nunits, a.G, a.topk, a.scale_log2, a.tile_info);
}

void launch_attn_dense(const LaunchAttnDense& a, hipStream_t st) {
  if (a.nunits <= 0) return;
  switch (a.bk) {
    case 128: launch_attn_dense_bk<128>(a, st); break;
    case 64: launch_attn_dense_bk<64>(a, st); break;
    case 32: launch_attn_dense_bk<32>(a, st); break;
    default: break;
  }
}

template <int BK>
static void launch_attn_decode_bk(const LaunchAttnDecode& a, hipStream_t st, int items) {
  hipLaunchKernelGGL(k_attn_decode<BK>, dim3(items), dim3(kDecWaves * 64), 0, st, a.q, a.k, a.v, a.ctx_lens,
                     a.sblk, a.nb, a.sel_out, a.out, a.lse_out, a.max_ctx, a.G, a.topk, a.scale_log2);
}

void launch_attn_decode(const LaunchAttnDecode& a, hipStream_t st) {
  const int items = a.batch * a.G;
  if (items <= 0) return;
  switch (a.bk) {
    case 128: launch_attn_decode_bk<128>(a, st, items); break;
    case 64: launch_attn_decode_bk<64>(a, st, items); break;
    case 32: launch_attn_decode_bk<32>(a, st, items); break;
    default: break;
  }
}

}  // namespace msa
