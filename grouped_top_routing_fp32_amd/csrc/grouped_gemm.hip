// Grouped expert GEMMs for batches with many rows per expert (prefill), gfx950.
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", its
// mixture-of-experts paragraph, and the Chinese translation of that post,
// 「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」, section 专家混合模型:
// each of the 8 experts a token is routed to is a SwiGLU MLP (hidden 5120,
// intermediate 2560); section 残差流 (residual stream): the SwiGLU product is
// computed in FP32.  Per expert e and
// routed row r (rows in expert-sorted order, tiles from the dispatch):
//   h[r] = silu(W_gate[e] x[r]) * (W_up[e] x[r])   bf16 MFMA, FP32 SwiGLU
//   y[r] = W_down[e] h[r]                           fp16 MFMA, FP32 accumulation
// h and y are stored as fp16 with a power-of-two scale 2^-s per (tile, 64
// columns), s chosen so the block's largest magnitude stays below 2^15.
//
// Block tile: 256 rows x 256 B-rows (gate/up: 128 gate + the same 128 up
// columns; down: 256 output columns), K advancing 64 per stage.  8 waves (two
// per SIMD) as 4 (rows) x 2 (columns); each wave owns 4 x 8 tiles of
// v_mfma_f32_16x16x32 (128 accumulators): row fragments 64 i + 16 wm, so a
// short tile drops whole levels i on every wave alike.
// When an expert's last tile has at most 64 rows (one level), the tile before
// it takes those rows as a fifth level (320 rows, 5 x 8 tiles per wave) and the
// last tile's blocks exit: the per-step copies and barrier of a one-level tile
// cost almost as much as a full one.  Both projections merge the same tiles, so
// a down tile is a gate/up tile and its per-stage activation scale is uniform.
//
// Memory: a stage's operand tiles (2 x 32 KB) are copied global -> LDS by the
// load unit (global_load_lds_dwordx4, no registers), each copy fetching 8 rows
// x 128 contiguous bytes (one cache line per row: half-line requests measured
// about 15% slower); two stages fit in LDS and stage t + 1 is requested at
// the start of step t.  Tiles of at most three levels keep three weight stages
// (and, at two levels, three activation stages) in the same 144 KB, with stage
// t + 2's weights requested at the start of step t: an expert with few rows
// streams its weights at a rate one stage of lead cannot sustain.  The copies
// are issued with inline assembly and waited for explicitly (s_waitcnt vmcnt,
// then s_barrier for the other waves): the compiler's own tracking of LDS
// copies adds a full drain at each loop head.
// Down: the weight stage is loaded into registers, converted to fp16 and
// written to LDS by the threads themselves, in the same layout the copies
// produce (on short tiles the copies bring the bf16 weights and each wave
// converts its own rows in place); the accumulators are kept in units of 2^s
// of the stage's 64-column activation block and rescaled (exactly) when s
// changes from one stage to the next, so the weights are never scaled.
// FP8 weights (E4M3 codes with one fp32 scale per output row; 「Reflection 放出
// 501B 的 Beam 权重：四套精度、滑动窗口和一场榜单落差」, the FP8 repository's
// precision listing): both projections take their weights through registers
// the same way, decoding 8 codes per lane exactly (bf16 for gate/up, fp16 for
// down); the row scales multiply the accumulators before the epilogue.
// Blocks are ordered for L2 reuse: each XCD (block b runs on XCD b % 8) takes
// a contiguous range of a linear order in which an expert's row tiles sweep
// the column blocks together, so blocks dispatched one after another share the
// weight columns or the row tile.
// LDS rows are 128 bytes; chunk c of row r sits at position c ^ ((r >> 1) & 7),
// so the 16 rows read by one MFMA operand load cover all 64 banks once.
#include <type_traits>

#include "common.h"

namespace beam {

namespace gg {

constexpr int kBM = 256;        // rows per tile
constexpr int kBN = 256;        // B-rows per tile
constexpr int kBK = 64;         // K per stage
constexpr int kThreads = 512;
constexpr int kSlotHalfs = kBM * kBK;  // 16384 elements = 32 KB per operand
// A tile followed by its expert's last tile, when that has at most kMergeRows
// rows, takes those rows too (kBM + kMergeRows rows, five levels): one block
// instead of two per column block.
constexpr int kMergeRows = 64;
constexpr int kRingHalfs = 2 * (kBM + kMergeRows + kBN) * kBK;  // 144 KB: two stages of 320 + 256 rows
static_assert(kBK == kScaleCols, "down reads one activation scale per stage");
static_assert(kBN == 4 * kScaleCols, "the down output tile spans four scale blocks");

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// XCD-aware order: block b runs on XCD b % 8; each XCD takes a contiguous
// range of the linear block order.
__device__ __forceinline__ int xcd_lin(int b, int total) {
  const int full = total & ~7;
  return b >= full ? b : (b & 7) * (full >> 3) + (b >> 3);
}

}  // namespace gg

// One block of a tile of at most 64 kLev rows (kLev row levels) against one
// column block; ring holds NA A stages of 64 kLev rows, then NB B stages.
// NB = 3 (tiles of at most three levels, operands copied by the load unit): the
// weights of two stages are in flight while the MFMAs consume a third.  Such
// tiles have few rows per weight byte and are bound by the weight stream, which
// one stage of lead leaves short of bytes in flight.  The activation rows (from
// L2, mostly) keep the same lead where a third A slot fits (NA = 3, two levels),
// else one stage (NA = 2).
template <bool GATEUP, bool FP8, int kLev, bool WF16, int NA = 2, int NB = 2>
__device__ __forceinline__ void gemm_block(uint16_t* ring, float* smax, int32_t* srow, uint8_t* stab, const Tile tl,
                                           int nblk, const uint16_t* __restrict__ act,
                                           const int32_t* __restrict__ sorted_slots, const void* __restrict__ w0v,
                                           const void* __restrict__ w1v, const float* __restrict__ s0,
                                           const float* __restrict__ s1, void* __restrict__ out,
                                           uint8_t* __restrict__ hscale, uint8_t* __restrict__ oscale, int Kdim,
                                           int Ndim, int topk) {
  using namespace gg;
  using WT = std::conditional_t<FP8, uint8_t, uint16_t>;  // weight element
  const WT* w0 = static_cast<const WT*>(w0v);
  const WT* w1 = static_cast<const WT*>(w1v);
  // weights through registers (FP8 codes, bf16 down weights to convert), or copied by the
  // load unit (bf16 gate/up weights, and down weights already in fp16: WF16)
  // bf16 down on the three-stage path: its weights are copied by the load unit as
  // bf16 and converted to fp16 in place in LDS, each wave its own 32 rows once they
  // have landed (the same conversion the register path applies)
  constexpr bool kCvtB = !GATEUP && !FP8 && !WF16 && NB == 3;
  constexpr bool kRegB = (FP8 || (!GATEUP && !WF16)) && !kCvtB;
  constexpr int BM = 64 * kLev;           // rows per A stage
  constexpr int kAPer = BM / 8;           // A rows copied per wave
  static_assert((NA == 2 && NB == 2) || (NB == 3 && NA >= 2 && NA <= 3 && !kRegB), "ring shapes");
  static_assert(!kCvtB || kBK * 2 * 32 == 4 * 64 * 16, "a wave's 32 weight rows are 4 KB: 4 chunks per lane");
  static_assert((NA * BM + NB * kBN) * kBK <= kRingHalfs, "ring");
  uint16_t(*sA)[BM * kBK] = reinterpret_cast<uint16_t(*)[BM * kBK]>(ring);
  uint16_t(*sB)[kSlotHalfs] = reinterpret_cast<uint16_t(*)[kSlotHalfs]>(ring + NA * BM * kBK);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // row fragments 64 i + 16 wm, i < kLev
  const int wn = wave & 1;   // column half
  const int BNc = GATEUP ? kBN / 2 : kBN;
  const int n0 = nblk * BNc;

  // ---- stage loads -----------------------------------------------------------
  // Wave w fills rows [kAPer w, kAPer (w + 1)) of the A slot and [32w, 32w+32) of
  // the B slot, 8 rows per 1 KB copy: lane i lands at byte 16 i, i.e. row + i/8,
  // position i%8, and so fetches chunk (i%8) ^ swz(row).
  const uint16_t* asrc[kLev];
  const WT* bsrc[4];
  {
    const WT* wbase = (GATEUP && wave >= 4 ? w1 : w0) + (size_t)tl.expert * Ndim * Kdim;  // B rows 128..: up
#pragma unroll
    for (int q = 0; q < kLev; ++q) {
      const int r = kAPer * wave + 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const int rr = min(r, tl.rows - 1);  // rows past the tile's end repeat its last row; never stored
      const size_t arow = GATEUP ? (size_t)(sorted_slots[tl.row_start + rr] / topk) : (size_t)(tl.row_start + rr);
      asrc[q] = act + arow * Kdim + c * 8;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 32 * wave + 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      bsrc[q] = wbase + (size_t)(n0 + (GATEUP ? (r & 127) : r)) * Kdim + c * 8;
    }
  }
  // A wave whose 32 rows all lie past the tile's end copies no activations: no MFMA
  // reads those LDS rows (a computed fragment starts below the tile's end, so its
  // rows are in the range of a wave that copies).  The main loop waits for all
  // copies at every step, so waves may issue different numbers of copies.
  if constexpr (!GATEUP)
    for (int r = tid; r < tl.rows; r += kThreads) srow[r] = sorted_slots[tl.row_start + r];
  const bool copy_a = kAPer * wave < tl.rows;
  auto issue_a = [&](int stage, int slot) {
    if (!copy_a) return;
    const int k = stage * kBK;
#pragma unroll
    for (int q = 0; q < kLev; ++q) lds_copy16(asrc[q] + k, lds_addr(&sA[slot][(kAPer * wave + 8 * q) * kBK]));
  };
  auto issue_b = [&](int stage, int slot) {
    const int k = stage * kBK;
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_copy16(bsrc[q] + k, lds_addr(&sB[slot][(32 * wave + 8 * q) * kBK]));
  };
  // Weights through registers (down, and every FP8 kernel): a lane loads the 8
  // weights of the chunk its copy would fetch (16 bytes of bf16 or 8 of E4M3 codes),
  // converts them and writes the 16 bytes where the copy would have put them.
  using BReg = std::conditional_t<FP8, uint2, u32x4>;
  BReg breg[4];
  const uint8_t* tscale = GATEUP ? nullptr : hscale + (size_t)tl.row_start * (Kdim / kScaleCols);
  // down: the stage's activation scale exponent is loaded with its weights, so
  // that its latency, like theirs, passes under the MFMAs of the current step
  int bsexp = 0;
  auto load_b = [&](int stage) {
    const int k = stage * kBK;
    if constexpr (!GATEUP) bsexp = tscale[stage];  // kBK == kScaleCols: one activation block per stage
#pragma unroll
    for (int q = 0; q < 4; ++q) breg[q] = *reinterpret_cast<const BReg*>(bsrc[q] + k);
  };
  // the weights are converted unscaled: down's accumulators carry the activations' 2^s
  auto convert_b = [&](int slot) {  // this wave's 32 rows of the slot, bf16 -> fp16 in place
    uint16_t* rows = &sB[slot][(32 * wave) * kBK];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4* c = reinterpret_cast<u32x4*>(rows + (lane + 64 * i) * 8);
      *c = bf16x8_to_f16x8(*c);
    }
  };
  auto store_b = [&](int slot) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 v;
      if constexpr (FP8) {
        const uint32_t c[2] = {breg[q].x, breg[q].y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if constexpr (GATEUP) {
            v[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false));
            v[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true));
          } else {
            v[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.0f, false));
            v[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.0f, true));
          }
        }
      } else {
        v = bf16x8_to_f16x8(breg[q]);
      }
      *reinterpret_cast<u32x4*>(&sB[slot][(32 * wave + 8 * q) * kBK + lane * 8]) = v;
    }
  };

  // ---- fragments and MFMAs -------------------------------------------------
  // Every fragment row is a multiple of 16 plus lane%16, so its chunk permutation
  // is swz(lane%16) throughout.  Sub-step s of a stage reads chunks 4s + lane/16.
  const int l16 = lane & 15;
  const int sw = swz(l16);
  const int fc = lane >> 4;
  const int aoff0 = (wm * 16 + l16) * kBK + ((fc ^ sw) << 3);
  const int aoff1 = (wm * 16 + l16) * kBK + (((4 + fc) ^ sw) << 3);
  const int brow = (GATEUP ? wn * 64 : wn * 128) + l16;
  const int boff0 = brow * kBK + ((fc ^ sw) << 3);
  const int boff1 = brow * kBK + (((4 + fc) ^ sw) << 3);
  const int nlev = min(kLev, (tl.rows - 16 * wm + 63) / 64);  // >= 0: levels with rows for this wave

  f32x4 acc[kLev][8];
#pragma unroll
  for (int i = 0; i < kLev; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto math = [&](int aslot, int bslot, int sub, auto full) {
    const uint16_t* A = sA[aslot];
    const uint16_t* B = sB[bslot];
    const int ao = sub ? aoff1 : aoff0;
    const int bo = sub ? boff1 : boff0;
    u32x4 fa[kLev], fb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // gate/up: j < 4 gate rows, j >= 4 the matching up rows (128 B-rows further)
      const int jj = GATEUP ? (j & 3) : j;
      const int extra = (GATEUP && j >= 4) ? 128 * kBK : 0;
      fb[j] = *reinterpret_cast<const u32x4*>(&B[bo + jj * 16 * kBK + extra]);
    }
#pragma unroll
    for (int i = 0; i < kLev; ++i) {
      if (decltype(full)::value || i < nlev) {
        fa[i] = *reinterpret_cast<const u32x4*>(&A[ao + i * 64 * kBK]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = GATEUP ? mfma16x16x32(fa[i], fb[j], acc[i][j]) : mfma16x16x32_f16(fa[i], fb[j], acc[i][j]);
      }
    }
  };

  // Gate/up takes both sub-steps of a stage at once: all 24 fragment reads, then the
  // 64 MFMAs, so the second half's reads overlap the first half's MFMAs (2% faster;
  // down, which also converts its weights, runs out of registers that way).
  auto math2 = [&](int slot, auto full) {
    const uint16_t* A = sA[slot];
    const uint16_t* B = sB[slot];
    u32x4 fa[2][4], fb[2][8];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ao = sub ? aoff1 : aoff0;
      const int bo = sub ? boff1 : boff0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        fb[sub][j] = *reinterpret_cast<const u32x4*>(&B[bo + (j & 3) * 16 * kBK + (j >= 4 ? 128 * kBK : 0)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (decltype(full)::value || i < nlev) fa[sub][i] = *reinterpret_cast<const u32x4*>(&A[ao + i * 64 * kBK]);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (decltype(full)::value || i < nlev) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(fa[sub][i], fb[sub][j], acc[i][j]);
        }
      }
  };

  // ---- main loop -----------------------------------------------------------
  // Stage t lives in slot t % 2.  Step t: wait for this wave's copies of stage t
  // (nothing later is in flight), barrier (stage t complete for all waves, and
  // everyone is done with the other slot), request stage t + 1 into the other
  // slot, MFMAs on stage t.  Weights through registers: stage t + 1's are loaded
  // before the MFMAs and written, converted, to the other slot after them; the
  // next barrier publishes them.
  const int nk = Kdim / kBK;  // Kdim % 128 == 0, so nk >= 2
  // down: the accumulators hold y * 2^-s_acc, s_acc the exponent of the last stage
  // consumed; s_next is the exponent of the stage waiting in the other slot
  int s_acc = 0, s_next = 0;
  if constexpr (NB == 2) {
    issue_a(0, 0);
    if constexpr (kRegB) {
      load_b(0);
      store_b(0);
    } else {
      issue_b(0, 0);
      if constexpr (!GATEUP) bsexp = tscale[0];
    }
    s_next = bsexp;
    s_acc = bsexp;
    auto main_loop = [&](auto full) {
      for (int st = 0; st < nk; ++st) {
        const int slot = st & 1;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        const bool more = st + 1 < nk;
        const int s_st = s_next;
        if (more) {
          issue_a(st + 1, slot ^ 1);
          if constexpr (kRegB) {
            load_b(st + 1);
          } else {
            issue_b(st + 1, slot ^ 1);
            if constexpr (!GATEUP) bsexp = tscale[st + 1];
          }
        }
        if constexpr (!GATEUP) {
          if (s_st != s_acc) {  // uniform: one exponent per tile and stage
#pragma unroll
            for (int i = 0; i < kLev; ++i)
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[i][j] = ldexp4(acc[i][j], s_acc - s_st);
            s_acc = s_st;
          }
        }
        if constexpr (GATEUP && !FP8 && kLev == 4) {
          math2(slot, full);
        } else {
          math(slot, slot, 0, full);
          math(slot, slot, 1, full);
        }
        if (more) {
          if constexpr (kRegB) store_b(slot ^ 1);
          s_next = bsexp;
        }
      }
    };
    // full tiles (the common case) run without the per-level tests
    if (tl.rows >= BM)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  } else {
    // Stage t's weights live in B slot t % 3 and its activations in A slot t % NA.
    // Step t: wait for this wave's copies of stage t (the later ones requested so
    // far, at most stage t + 1's, may still be in flight), barrier (stage t complete
    // for all waves, and everyone is done with stage t - 1's slots), request the
    // activations of stage t + NA - 1 and the weights of stage t + 2 into the slots
    // stage t - 1 held, MFMAs on stage t.  Requests go out in stage order per wave,
    // so waiting until only the copies issued after stage t's remain is enough: with
    // NA = 3 those are all of stage t + 1's, with NA = 2 its weight copies (4).
    // Down reads each stage's activation scale exponent from the tile's table in LDS
    // (stab, filled before the first barrier).
    const int ncopies = (copy_a ? kLev : 0) + 4;  // copies per stage issued by this wave
    if constexpr (!GATEUP)
      for (int i = tid; i < nk; i += kThreads) stab[i] = tscale[i];
    issue_a(0, 0);
    issue_b(0, 0);
    if constexpr (NA == 3) issue_a(1, 1);
    issue_b(1, 1);
    if constexpr (kCvtB) {
      // stage 0's weights: issued before stage 1's copies (and, NA = 3, stage 1's activations)
      if (NA == 3 && copy_a)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLev + 4));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
      asm volatile("" ::: "memory");
      convert_b(0);
    }
    auto main_loop3 = [&](auto full) {
      for (int st = 0; st < nk; ++st) {
        const int slot = st % 3;
        if (st + 1 == nk)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else if (NA == 3 && ncopies == kLev + 4)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLev + 4));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        if (st + NA - 1 < nk) issue_a(st + NA - 1, (st + NA - 1) % NA);
        if (st + 2 < nk) issue_b(st + 2, (st + 2) % 3);
        if constexpr (!GATEUP) {
          const int s_st = stab[st];
          if (s_st != s_acc) {  // uniform: one exponent per tile and stage
#pragma unroll
            for (int i = 0; i < kLev; ++i)
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[i][j] = ldexp4(acc[i][j], s_acc - s_st);
            s_acc = s_st;
          }
        }
        math(st % NA, slot, 0, full);
        math(st % NA, slot, 1, full);
        if constexpr (kCvtB) {
          // stage st + 1's weights (requested a step earlier) into fp16 for the next step;
          // requested after them: this step's activation and weight copies
          if (st + 1 < nk) {
            const bool a_later = st + NA - 1 < nk && copy_a, b_later = st + 2 < nk;
            if (a_later && b_later)
              __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLev + 4));
            else if (b_later)
              __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
            else if (a_later)
              __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLev));
            else
              __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            asm volatile("" ::: "memory");
            convert_b((st + 1) % 3);
          }
        }
      }
    };
    if (tl.rows >= BM)
      main_loop3(std::true_type{});
    else
      main_loop3(std::false_type{});
  }

  // ---- epilogue ----------------------------------------------------------
  // lane holds rows 4*(lane/16)+r and column lane%16 of each 16x16 block
  // FP8: the row scales of this lane's columns (gate/up: the gate and up rows of column
  // n0 + wn*64 + 16 j + lane%16; down: output column n0 + wn*128 + 16 j + lane%16)
  float rs[8];
  if constexpr (FP8) {
    const size_t sb = (size_t)tl.expert * Ndim + n0 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rs[j] = GATEUP ? (j < 4 ? s0 : s1)[sb + wn * 64 + 16 * (j & 3)] : s0[sb + wn * 128 + 16 * j];
#pragma unroll
    for (int i = 0; i < kLev; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] *= rs[j];
  }
  if (!GATEUP && s_acc != 0) {  // y = acc * 2^s_acc
#pragma unroll
    for (int i = 0; i < kLev; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = ldexp4(acc[i][j], s_acc);
  }
  if (GATEUP) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < kLev; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = 64 * i + 16 * wm + (lane >> 4) * 4 + r < tl.rows;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = ok ? silu_f32(acc[i][j][r]) * acc[i][4 + j][r] : 0.f;
          acc[i][j][r] = v;
          mx = fmaxf(mx, fabsf(v));
        }
      }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    float bm = smax[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) bm = fmaxf(bm, smax[w]);
    const int sexp = act_scale_exp(bm);
    const int nsb = Ndim / kScaleCols;
    for (int r = tid; r < tl.rows; r += kThreads)
#pragma unroll
      for (int b = 0; b < 128 / kScaleCols; ++b)
        hscale[(size_t)(tl.row_start + r) * nsb + n0 / kScaleCols + b] = (uint8_t)sexp;
#pragma unroll
    for (int i = 0; i < kLev; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 64 * i + 16 * wm + (lane >> 4) * 4 + r;
        if (row < tl.rows) {
          uint16_t* hrow = reinterpret_cast<uint16_t*>(out) + (size_t)(tl.row_start + row) * Ndim + n0 + wn * 64 +
                           (lane & 15);
#pragma unroll
          for (int j = 0; j < 4; ++j) hrow[16 * j] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(acc[i][j][r], -sexp));
        }
      }
  } else {
    // Output tile as fp16 scaled by 2^-s per 64 columns, s from the tile's largest
    // magnitude in those columns.  Wave (wm, wn) holds columns wn*128 + 16 j +
    // lane%16, i.e. the 64-column blocks 2 wn (j < 4) and 2 wn + 1 (j >= 4).
    // (Staging the tile in LDS to store whole rows measured slower.)
    float mx[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kLev; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = 64 * i + 16 * wm + (lane >> 4) * 4 + r < tl.rows;
#pragma unroll
        for (int j = 0; j < 8; ++j) mx[j >> 2] = fmaxf(mx[j >> 2], ok ? fabsf(acc[i][j][r]) : 0.f);
      }
    mx[0] = wave_max(mx[0]);
    mx[1] = wave_max(mx[1]);
    if (lane == 0) {
      smax[2 * wave] = mx[0];
      smax[2 * wave + 1] = mx[1];
    }
    __syncthreads();
    // scale of 64-column block b = 2 wn' + half: max over the four row waves wm'
    auto block_exp = [&](int b) {
      float m = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) m = fmaxf(m, smax[2 * ((w2 << 1) | (b >> 1)) + (b & 1)]);
      return act_scale_exp(m);
    };
    const int sexp0 = block_exp(2 * wn), sexp1 = block_exp(2 * wn + 1);
    uint16_t* y16 = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int i = 0; i < kLev; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 64 * i + 16 * wm + (lane >> 4) * 4 + r;
        if (row < tl.rows) {
          uint16_t* yrow = y16 + (size_t)srow[row] * Ndim + n0 + wn * 128 + (lane & 15);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            yrow[16 * j] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(acc[i][j][r], -(j < 4 ? sexp0 : sexp1)));
        }
      }
    const int nsb = Ndim / kScaleCols;
    for (int q = tid; q < tl.rows * 4; q += kThreads) {
      const int row = q >> 2, b = q & 3;
      oscale[(size_t)srow[row] * nsb + n0 / kScaleCols + b] = (uint8_t)block_exp(b);
    }
  }
}

// GATEUP: act = x [T, H]; w0 = W_gate, w1 = W_up [E, I, H]; out = h fp16 [n, I]; hscale written.
// !GATEUP: act = h fp16 [n, I]; w0 = W_down [E, H, I]; hscale read; out = y fp16 [n, H] (row slot),
//          scaled by 2^-s with s per (tile, 64 columns) written to oscale [n, H / 64].
// FP8: the weights are E4M3 codes (uint8) with one fp32 scale per output row (s0 for w0, s1 for
//      w1, [E, Ndim]); every copy of them passes through registers, where the codes are decoded
//      exactly (to bf16 for gate/up, to fp16 for down), and the row scales multiply the
//      accumulators before the epilogue.
template <bool GATEUP, bool FP8, bool WF16 = false>
__global__ __launch_bounds__(gg::kThreads, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ sorted_slots, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const void* __restrict__ w0v, const void* __restrict__ w1v,
    const float* __restrict__ s0, const float* __restrict__ s1, void* __restrict__ out,
    uint8_t* __restrict__ hscale, uint8_t* __restrict__ oscale, int Kdim, int Ndim, int topk, int nbn,
    int total_blocks) {
  using namespace gg;
  // two stages of A, then two of B
  __shared__ __attribute__((aligned(16))) uint16_t ring[kRingHalfs];
  __shared__ float smax[16];
  // down: destination slots of the tile's rows, read when the block starts so that the
  // epilogue's stores need no dependent global loads
  __shared__ int32_t srow[GATEUP ? 1 : kBM + kMergeRows];
  // down, three-stage tiles: the tile's activation scale exponent per stage (Kdim <= 32768)
  __shared__ uint8_t stab[GATEUP ? 1 : 512];

  // The grid is sized for the most tiles a batch can have; the order spans the
  // tiles this batch has, so every XCD gets an equal share and the surplus
  // blocks (the highest indices) exit here.  Linear order: tile group by tile
  // group (an expert's tiles, at most kTileGroupMax), inside a group column
  // block by column block, the group's tiles in snake order, so consecutive
  // blocks share either the weight columns or (at each turn) the row tile.
  const int nt = ntiles[0];
  const int real_blocks = min(total_blocks, nt * nbn);
  if ((int)blockIdx.x >= real_blocks) return;
  const int lin = xcd_lin(blockIdx.x, real_blocks);
  const Tile tg = tiles[lin / nbn];  // a tile of the block's group
  const int r = lin - nbn * tg.group_first;
  const int nblk = r / tg.group_size;
  int j = r - nblk * tg.group_size;
  if (nblk & 1) j = tg.group_size - 1 - j;
  const int idx = tg.group_first + j;
  Tile tl = tiles[idx];
  {
    // Only an expert's last tile can be short, and the tile before it has kBM
    // rows, so a merged tile has at most kBM + kMergeRows rows.
    const Tile prev = tiles[max(idx - 1, 0)];
    const Tile next = tiles[min(idx + 1, nt - 1)];
    if (idx > 0 && prev.expert == tl.expert && tl.rows <= kMergeRows) return;  // merged into the tile before
    if (idx + 1 < nt && next.expert == tl.expert && next.rows <= kMergeRows) {
      tl.rows += next.rows;
      gemm_block<GATEUP, FP8, (kBM + kMergeRows) / 64, WF16>(ring, smax, srow, stab, tl, nblk, act, sorted_slots,
                                                             w0v, w1v, s0, s1, out, hscale, oscale, Kdim, Ndim, topk);
      return;
    }
  }
  // Tiles of at most three levels (experts with few rows) are bound by their
  // weight stream: where the load unit copies the weights (bf16 gate/up, fp16 down,
  // and bf16 down, converted in LDS) they keep two stages of them in flight.  (The
  // FP8 kernels, which decode their weights through registers, are bound by their
  // LDS traffic at these heights, not by the stream.)
  if constexpr (!FP8) {
    if (tl.rows <= 128) {
      gemm_block<GATEUP, FP8, 2, WF16, 3, 3>(ring, smax, srow, stab, tl, nblk, act, sorted_slots, w0v, w1v, s0, s1,
                                             out, hscale, oscale, Kdim, Ndim, topk);
      return;
    }
    if (tl.rows <= 192) {
      gemm_block<GATEUP, FP8, 3, WF16, 2, 3>(ring, smax, srow, stab, tl, nblk, act, sorted_slots, w0v, w1v, s0, s1,
                                             out, hscale, oscale, Kdim, Ndim, topk);
      return;
    }
  }
  gemm_block<GATEUP, FP8, kBM / 64, WF16>(ring, smax, srow, stab, tl, nblk, act, sorted_slots, w0v, w1v, s0, s1, out,
                                          hscale, oscale, Kdim, Ndim, topk);
}

int grouped_gemm_rows() { return gg::kBM; }

static int gemm_blocks(int max_tiles, int nbn) { return max_tiles * nbn; }

hipError_t launch_gateup_grouped(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                 int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale,
                                 int H, int I, int K, hipStream_t st) {
  const int nbn = I / (gg::kBN / 2);  // I % 128 == 0
  const int total = gemm_blocks(max_tiles, nbn);
  hipLaunchKernelGGL((grouped_gemm_kernel<true, false>), dim3(total), dim3(gg::kThreads), 0, st, x, slots, tiles,
                     ntiles, wg, wu, nullptr, nullptr, (void*)h, hscale, nullptr, H, I, K, nbn, total);
  return hipGetLastError();
}

// wd_f16: W_down already converted to fp16 (beam_moe_pack_weights): copied into LDS by
// the load unit like the gate/up weights, with no conversion.
hipError_t launch_down_grouped(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                               const int32_t* ntiles, int max_tiles, const uint16_t* wd, bool wd_f16, uint16_t* y16,
                               uint8_t* yscale, int H, int I, hipStream_t st) {
  const int nbn = H / gg::kBN;  // H % 256 == 0
  const int total = gemm_blocks(max_tiles, nbn);
  if (wd_f16)
    hipLaunchKernelGGL((grouped_gemm_kernel<false, false, true>), dim3(total), dim3(gg::kThreads), 0, st, h, slots,
                       tiles, ntiles, wd, nullptr, nullptr, nullptr, (void*)y16, const_cast<uint8_t*>(hscale), yscale,
                       I, H, 0, nbn, total);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<false, false>), dim3(total), dim3(gg::kThreads), 0, st, h, slots, tiles,
                       ntiles, wd, nullptr, nullptr, nullptr, (void*)y16, const_cast<uint8_t*>(hscale), yscale, I, H,
                       0, nbn, total);
  return hipGetLastError();
}

hipError_t launch_gateup_grouped_fp8(const uint16_t* x, const int32_t* slots, const Tile* tiles,
                                     const int32_t* ntiles, int max_tiles, const uint8_t* wg, const uint8_t* wu,
                                     const float* sg, const float* su, uint16_t* h, uint8_t* hscale, int H, int I,
                                     int K, hipStream_t st) {
  const int nbn = I / (gg::kBN / 2);
  const int total = gemm_blocks(max_tiles, nbn);
  hipLaunchKernelGGL((grouped_gemm_kernel<true, true>), dim3(total), dim3(gg::kThreads), 0, st, x, slots, tiles,
                     ntiles, wg, wu, sg, su, (void*)h, hscale, nullptr, H, I, K, nbn, total);
  return hipGetLastError();
}

hipError_t launch_down_grouped_fp8(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                                   const int32_t* ntiles, int max_tiles, const uint8_t* wd, const float* sd,
                                   uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st) {
  const int nbn = H / gg::kBN;
  const int total = gemm_blocks(max_tiles, nbn);
  hipLaunchKernelGGL((grouped_gemm_kernel<false, true>), dim3(total), dim3(gg::kThreads), 0, st, h, slots, tiles,
                     ntiles, wd, nullptr, sd, nullptr, (void*)y16, const_cast<uint8_t*>(hscale), yscale, I, H, 0,
                     nbn, total);
  return hipGetLastError();
}

}  // namespace beam
