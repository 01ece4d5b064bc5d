// Hessian statistics S += X^T X for token-major activations X [n_tok, d].
//
// [derivation] eq. (9): H = (2/N) X X^T with X = reshape(A, [N, d])^T
// (eq. (5)); the sum is additive over calibration chunks (section 9.4).
// The statistic is symmetric, so only the upper triangle is computed and
// the result is mirrored.
//
// bf16 path (the hot path): one workgroup of eight wave64s (two per SIMD,
// so one wave's LDS waits and barriers overlap the other's MFMAs) per
// (256x256 upper super-tile of S, token split); wave w owns the 128x64
// half h = w % 2 of the 128x128 sub-tile (q / 2, q % 2), q = w / 2, and its
// 128 fp32 accumulators sit in the AGPRs.  The two 256-feature panels of
// each 32-token step are staged once per workgroup in LDS and shared by the
// eight waves.
//  * Unmasked items: global_load_lds_dwordx4 copies the token rows straight
//    into a four-stage LDS ring (loads run three steps ahead, no VGPRs), and
//    ds_read_b64_tr_b16 transposes them into v_mfma_f32_16x16x32_bf16
//    operands on the way out.
//  * Masked items (a panel crossing d, a ragged last split): each thread
//    gathers an 8-token x 8-feature block with 16-byte loads, zeroes what
//    lies outside, transposes it in registers (v_perm_b32) and writes it
//    feature-major into a double-buffered LDS stage.
// bf16 x bf16 products are exact in fp32 and accumulate in fp32.  Token
// splits write fp32 partial tiles that a second kernel adds to S in split
// order with an fp64 running sum (bitwise reproducible).
//
// fp32 path: plain tiled kernel accumulating in fp64 (small inputs).
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int kSup = 256;                      // super-tile edge (features)
constexpr int kStep = 32;                      // tokens per step
constexpr int kThreads = 512;                  // eight wave64s
constexpr int kPanelBytes = 4 * kSup * 16;     // 4 token chunks x 256 features x 16 B
constexpr int kStageBytes = 2 * kPanelBytes;
constexpr int kLdsBytes = 2 * kStageBytes;     // two stages: 64 KiB
constexpr int kSubElems = 128 * 128;           // one 128x128 sub-tile's partial
constexpr int kCUs = 256;                      // MI355X compute units
constexpr int kXcd = 8;                        // accelerator dies, own L2 each
constexpr int kRegB = 8;                       // work order: blocks of 8x8 super-tiles
constexpr int64_t kMaxChain = 2048;            // steps per fp32 running sum (see plan_splits)

__host__ __device__ inline int64_t upper_tiles(int64_t nt) { return nt * (nt + 1) / 2; }

__device__ inline void tile_of(int64_t L, int nt, int& ti, int& tj) {
  int t = 0;
  int64_t rem = L;
  while (rem >= nt - t) {
    rem -= nt - t;
    ++t;
  }
  ti = t;
  tj = t + static_cast<int>(rem);
}

// XCD-aware work order.  The work items (super-tile, token split) form one
// list, split-major, and within a split the upper super-tiles are enumerated
// block-major (blocks of kRegB x kRegB, row-major over the upper block
// triangle, row-major inside a block).  Workgroup w runs on XCD w % 8, in
// dispatch order within its XCD, and XCD x takes the x-th contiguous eighth
// of the list.  The workgroups one XCD runs at a time therefore read the same
// token window of a compact set of panels (a triangle of side 8 or a 4 x 8
// rectangle of super-tiles touches 8 or 12 of them), which its L2 serves.
__device__ inline void blocked_tile(int64_t t, int nt, int& ti, int& tj) {
  const int nb = (nt + kRegB - 1) / kRegB;
  for (int br = 0; br < nb; ++br) {
    const int r0 = br * kRegB, rh = min(kRegB, nt - r0);
    for (int bc = br; bc < nb; ++bc) {
      const int c0 = bc * kRegB, cw = min(kRegB, nt - c0);
      const int64_t size = (bc == br) ? int64_t(rh) * (rh + 1) / 2 : int64_t(rh) * cw;
      if (t >= size) {
        t -= size;
        continue;
      }
      if (bc == br) {
        int i = 0;
        while (t >= rh - i) {
          t -= rh - i;
          ++i;
        }
        ti = r0 + i;
        tj = r0 + i + static_cast<int>(t);
      } else {
        ti = r0 + static_cast<int>(t / cw);
        tj = c0 + static_cast<int>(t % cw);
      }
      return;
    }
  }
  ti = tj = 0;
}

// Row-major index of upper super-tile (ti, tj) (the partial-sum layout).
__device__ inline int64_t upper_index(int ti, int tj, int nt) {
  return int64_t(ti) * nt - int64_t(ti) * (ti - 1) / 2 + (tj - ti);
}

// Loader geometry of the masked path: thread t fetches panel t / 128 (0:
// rows F0.., 1: columns G0..), features 8*fg .. 8*fg+7 with fg = t % 32,
// tokens 8*tg .. 8*tg+7 of the step with tg = (t / 32) % 4; raw[q] holds
// token 8*tg + q.
//
// Ragged steps (token tail, or a panel crossing d; needs d % 8 == 0 so a
// lane's 8 features are all in range or all out): out-of-range tokens and
// features read a clamped in-range address and are zeroed.
__device__ inline void load_masked(const uint16_t* __restrict__ X, int64_t ldx,
                                   int64_t tb, int64_t t0, int64_t tend,
                                   int64_t f, int64_t d, u32x4 raw[8]) {
  const bool fv = f < d;
  const int64_t fc = fv ? f : 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bool tv = tb + q < tend;
    const u32x4 v = *reinterpret_cast<const u32x4*>(X + (tv ? tb + q : t0) * ldx + fc);
    raw[q] = (fv && tv) ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

// raw[q].dword[p] = features (2p, 2p+1) of token q  ->
// frag[f].dword[t] = tokens (2t, 2t+1) of feature f.  One v_perm_b32 per
// output dword: bytes 0-3 of the selector index the second operand (token
// 2t), bytes 4-7 the first (token 2t+1).
__device__ inline void transpose8x8(const u32x4 raw[8], u32x4 frag[8]) {
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      o[t] = __builtin_amdgcn_perm(raw[2 * t + 1][f >> 1], raw[2 * t][f >> 1], sel);
    frag[f] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// LDS layout of one panel in one stage: 16-byte units (token chunk c = 0..3,
// feature r = 0..255) at unit index c * 256 + (r ^ ((r >> 3) & 15)).  The XOR
// keeps both access patterns free of bank conflicts: the loader's writes
// (rows 8*fg + f for 16 consecutive fg) and the MFMA reads (16 consecutive
// rows of one chunk) each touch 16 distinct 16-byte bank groups.
__device__ inline uint32_t lds_unit(int c, int r) {
  return static_cast<uint32_t>((c * kSup + (r ^ ((r >> 3) & 15))) * 16);
}

__device__ inline void store_panel(char* lds, uint32_t panel_off, int fg, int tg,
                                   const u32x4 raw[8]) {
  u32x4 frag[8];
  transpose8x8(raw, frag);
#pragma unroll
  for (int f = 0; f < 8; ++f)
    *reinterpret_cast<u32x4*>(lds + panel_off + lds_unit(tg, 8 * fg + f)) = frag[f];
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup barrier between LDS stages.  Only LDS traffic is waited for: the
// global loads of the steps ahead stay in flight across it.
__device__ inline void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc += A B on v_mfma_f32_16x16x32_bf16 with the accumulator pinned to the
// AGPR file: left to itself the register allocator shuttles accumulators
// between the two files (and to scratch) once the staging registers are
// counted.
// Consecutive MFMAs of a step use distinct accumulators; after the last
// step acc_settle() covers the wait states before the results are read.
__device__ inline void mfma_acc(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ inline void acc_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// One 32-token step of a wave: 8 + 4 fragment reads, 8 x 4 MFMAs.
// acc[a][b] lane l element v = sum over the step's tokens of
// x[row 16a + 4(l/16) + v] * x[col 16b + l%16] within the wave's 128x64
// tile.  The B fragments and the first two A fragments are read up front;
// A fragment a + 2 is read while the MFMAs of row block a run.
__device__ inline void mma_step(const char* lds, uint32_t a_off, uint32_t b_off,
                                const uint32_t offA[8], const uint32_t offB[4],
                                f32x4 acc[8][4]) {
  u32x4 fa[8], fb[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
    fb[b] = *reinterpret_cast<const u32x4*>(lds + b_off + offB[b]);
  fa[0] = *reinterpret_cast<const u32x4*>(lds + a_off + offA[0]);
  fa[1] = *reinterpret_cast<const u32x4*>(lds + a_off + offA[1]);
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    if (a + 2 < 8) fa[a + 2] = *reinterpret_cast<const u32x4*>(lds + a_off + offA[a + 2]);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      mfma_acc(acc[a][b], fa[a], fb[b]);
    }
  }
}

// The step loop of a masked work item (a panel crossing d, or a ragged last
// split): register-staged loads with zeros outside the data, the step count
// padded to even with all-zero steps; loads of the steps past the end
// re-read the last step.
// The first four waves load and store the stages; all eight compute.
__device__ inline void run_masked(char* lds, const uint16_t* __restrict__ X,
                                 int64_t ldx, int64_t d, int64_t tbeg,
                                 int64_t tend, int64_t P0, uint32_t b_panel, const uint32_t offA[8],
                                 const uint32_t offB[4], f32x4 acc[8][4]) {
  const int tid = threadIdx.x;
  const bool loader = tid < 256;
  const int lp = (tid >> 7) & 1, fg = tid & 31, tg = (tid >> 5) & 3;
  const uint32_t panel_off = static_cast<uint32_t>(lp) * kPanelBytes;
  const int64_t nst = (tend - tbeg + kStep - 1) / kStep;
  const int64_t nst2 = (nst + 1) & ~int64_t(1);
  auto load_step = [&](int64_t s, u32x4 raw[8]) {
    if (!loader) return;
    s = s < nst2 ? s : nst2 - 1;
    const int64_t t0 = tbeg + s * kStep;
    load_masked(X, ldx, t0 + 8 * tg, tbeg, tend, P0 + 8 * fg, d, raw);
  };
  auto store = [&](uint32_t off, const u32x4 raw[8]) {
    if (loader) store_panel(lds, off + panel_off, fg, tg, raw);
  };
  // LDS stage k % 2 holds step k; raw0 / raw1 carry the loads of the even /
  // odd step ahead, two steps before their use.
  u32x4 raw0[8], raw1[8];
  load_step(0, raw0);
  load_step(1, raw1);
  store(0, raw0);
  stage_barrier();
  for (int64_t s = 0; s < nst2; s += 2) {
    load_step(s + 2, raw0);
    mma_step(lds, 0, b_panel, offA, offB, acc);
    store(kStageBytes, raw1);
    stage_barrier();
    load_step(s + 3, raw1);
    mma_step(lds, kStageBytes, kStageBytes + b_panel, offA, offB, acc);
    store(0, raw0);
    stage_barrier();
  }
}

// ---------------------------------------------------------------------------
// Unmasked items: direct-to-LDS staging.  Each step's two panels (32 token
// rows x 256 features each) go from global memory straight into LDS with
// global_load_lds_dwordx4 (no VGPRs, no transposes), token-major, in a ring
// of kStages stages, so the loads run kStages - 1 steps ahead of the MFMAs.
// The MFMA operands are read with ds_read_b64_tr_b16, which transposes
// within 16-lane groups: lane i of a group receives element i % 4 of the
// 8-byte reads of lanes 4e + i / 4 (e = 0..3).  A lane group that points
// lanes 4e + m at token row R + e, features F + 4m .. F + 4m + 3 thus gives
// lane i the features F + i of tokens R .. R + 3 -- half an MFMA fragment.
// ---------------------------------------------------------------------------
constexpr int kStages = 4;
constexpr int kRowBytes = kSup * 2;                    // one token row of a panel
constexpr int kDmaPanel = kStep * kRowBytes;           // 16 KiB
constexpr int kDmaStage = 2 * kDmaPanel;               // 32 KiB

// 16-byte chunk c of token row r is stored at chunk c ^ swz(r).  Each
// ds_read_b64_tr_b16 reads, per half-wave, 32 bytes from each of 8 rows
// whose swz values differ in bits 1-3, so the 8 reads cover the 64 banks
// once.
__device__ inline int swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef const void __attribute__((address_space(1)))* gvoid;
typedef void __attribute__((address_space(3)))* lvoid;

__device__ inline uint2 tr_read(const char* lds, uint32_t off) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds + off));
  return __builtin_bit_cast(uint2, v);
}

// Fragment: tokens 8*kg + e (from h = 0) and 8*kg + 4 + e (h = 1, four rows
// = 2048 bytes further) of feature column `off` addresses.
__device__ inline u32x4 tr_frag(const char* lds, uint32_t off) {
  const uint2 lo = tr_read(lds, off), hi = tr_read(lds, off + 4 * kRowBytes);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

template <int n>
__device__ inline void wait_vmcnt_le() {
  // s_waitcnt with vmcnt = n (split field), expcnt and lgkmcnt at maximum
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline void run_dma(char* lds, const uint16_t* __restrict__ X,
                               int64_t ldx, int64_t tbeg, int64_t nst,
                               int64_t F0, int64_t G0, f32x4 acc[8][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // loader role: wave wv fills panel wv / 4, rows 8 (wv % 4) + 2 i + lane / 32
  // (instruction i = 0..3); lanes write 16 contiguous bytes each
  const int p = wv >> 2;
  const int64_t P0 = p ? G0 : F0;
  uint32_t goff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (wv & 3) + 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ swz(r);
    goff[i] = static_cast<uint32_t>(2 * (r * ldx + P0 + 8 * c));
  }
  const uint32_t lds_row0 = static_cast<uint32_t>(p * kDmaPanel + 8 * (wv & 3) * kRowBytes);
  // MFMA role: half h of sub-tile (wa, wb); lane (kg, j) points at row
  // 8 kg + j / 4, features 4 (j % 4) .. + 3 of each 16-feature block
  const int q = wv >> 1, h = wv & 1;
  const int wa = q >> 1, wb = q & 1;
  const int kg = lane >> 4, j = lane & 15;
  const int r0 = 8 * kg + (j >> 2);
  const int sw = swz(r0);
  uint32_t aoff[8], boff[4];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int cl = 2 * a + ((j & 3) >> 1);
    aoff[a] = static_cast<uint32_t>(r0 * kRowBytes + 16 * ((16 * wa + cl) ^ sw) + 8 * (j & 1));
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int cl = 2 * (4 * h + b) + ((j & 3) >> 1);
    boff[b] = static_cast<uint32_t>(kDmaPanel + r0 * kRowBytes + 16 * ((16 * wb + cl) ^ sw) + 8 * (j & 1));
  }

  // load i of step k (token rows 2i, 2i + 1 of this wave's quarter panel)
  auto src_of = [&](int64_t k) {
    const int64_t kk = k < nst ? k : nst - 1;
    const uint16_t* base = X + (tbeg + kk * kStep) * ldx;
    asm volatile("" : "+s"(base));
    return reinterpret_cast<const char*>(base);
  };
  auto dst_of = [&](int slot) {
    return lds + static_cast<uint32_t>(slot) * kDmaStage + lds_row0;
  };

#pragma unroll
  for (int k = 0; k < kStages - 1; ++k) {
    const char* gb = src_of(k);
    char* dst = dst_of(k);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((gvoid)(gb + goff[i]), (lvoid)(dst + 2 * i * kRowBytes),
                                       16, 0, 0);
  }
  wait_vmcnt_le<4 * (kStages - 2)>();
  stage_barrier();
  // Each step is two halves (row blocks 0-3, 4-7) ending in a barrier.  The
  // second wave of each SIMD (waves 4-7) runs one half behind the first:
  // after every barrier one of a SIMD's two waves starts a step (fragment
  // reads first) while the other is in its second half, whose first
  // fragments it read before the barrier, and keeps the MFMA pipe busy.
  // Ordering of the ring under this skew: the loads of step s + 3 go out in
  // the second half of step s, when both waves are done with step s - 1
  // (the slot they refill); each wave waits for its loads of step s + 1 at
  // the end of the first half of step s, before the barrier after which the
  // leading waves start reading it.
  const bool late = wv >= 4;
  if (late) stage_barrier();
  // ring slots of step s and of step s + kStages - 1 (the slot before it)
  int cur = 0, ahead = kStages - 1;
  for (int64_t s = 0; s < nst; ++s) {
    const char* gb = src_of(s + kStages - 1);
    char* dst = dst_of(ahead);
    const char* st = lds + static_cast<uint32_t>(cur) * kDmaStage;
    ahead = cur;
    cur = (cur + 1 == kStages) ? 0 : cur + 1;
    u32x4 fa[8], fb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) fb[b] = tr_frag(st, boff[b]);
    fa[0] = tr_frag(st, aoff[0]);
    fa[1] = tr_frag(st, aoff[1]);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        mfma_acc(acc[a][b], fa[a], fb[b]);
        if (b == 1 && a >= 4)
          __builtin_amdgcn_global_load_lds((gvoid)(gb + goff[a - 4]),
                                           (lvoid)(dst + 2 * (a - 4) * kRowBytes), 16, 0, 0);
        if (b == 2 && a + 2 < 8) fa[a + 2] = tr_frag(st, aoff[a + 2]);
      }
      if (a == 3) {
        wait_vmcnt_le<4 * (kStages - 3)>();
        stage_barrier();
      }
    }
    stage_barrier();
  }
  // as many barriers for every wave; after this one no wave reads the ring
  if (!late) stage_barrier();
  // the loads issued past the last step (they re-read it) land before the
  // workgroup's LDS is released
  wait_vmcnt_le<0>();
}

// kFull selects the work items this instance runs: the unmasked ones (both
// panels inside [0, d), an even number of full steps) or the rest; the host
// launches the masked instance only when such items exist.  Separate
// instances keep the masked loop's registers out of the hot loop.
template <bool kFull>
__global__ __launch_bounds__(kThreads) void hessian_bf16_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t n_tok, int64_t d,
    int nt, int64_t ks, int nsplit, float* __restrict__ S,
    float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char lds[kFull ? kStages * kDmaStage : kLdsBytes];
  // work item of this workgroup (see blocked_tile)
  const int64_t ntiles = upper_tiles(nt);
  const int64_t nitems = ntiles * nsplit;
  // rounds of kCUs workgroups take consecutive runs of the list, XCD x the
  // x-th run of kCUs / kXcd items of each round
  const int64_t w = blockIdx.x;
  constexpr int64_t kPer = kCUs / kXcd;
  const int64_t item = (w / kCUs) * kCUs + (w % kXcd) * kPer + (w / kXcd) % kPer;
  if (item >= nitems) return;
  const int split = static_cast<int>(item / ntiles);
  const int64_t t = item % ntiles;
  int ti, tj;
  blocked_tile(t, nt, ti, tj);
  const bool diag = ti == tj;
  const int64_t F0 = int64_t(ti) * kSup, G0 = int64_t(tj) * kSup;
  const int64_t tbeg = int64_t(split) * ks;
  const int64_t tend = min(tbeg + ks, n_tok);
  const int64_t ntok = tend - tbeg;
  const bool full = (F0 + kSup <= d) && (G0 + kSup <= d) && ntok % kStep == 0;
  if (full != kFull) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  // Masked loader role: threads 0-127 stage the row panel, 128-255 the
  // column panel (on a diagonal super-tile both hold the same features).
  const int64_t P0 = ((tid >> 7) & 1) ? G0 : F0;
  // MFMA role: wave wv owns half h of sub-tile q = (wa, wb).  On a diagonal
  // super-tile the lower sub-tile (1, 0) mirrors (0, 1): it is computed
  // (keeping the step free of branches) but not written.
  const int q = wv >> 1, h = wv & 1;
  const int wa = q >> 1, wb = q & 1;
  const bool busy = !(diag && q == 2);
  const int c = lane >> 4, i16 = lane & 15;
  uint32_t offA[8], offB[4];
#pragma unroll
  for (int a = 0; a < 8; ++a) offA[a] = lds_unit(c, 128 * wa + 16 * a + i16);
#pragma unroll
  for (int b = 0; b < 4; ++b) offB[b] = lds_unit(c, 128 * wb + 64 * h + 16 * b + i16);
  const uint32_t b_panel = static_cast<uint32_t>(kPanelBytes);

  f32x4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kFull)
    run_dma(lds, X, ldx, tbeg, ntok / kStep, F0, G0, acc);
  else
    run_masked(lds, X, ldx, d, tbeg, tend, P0, b_panel, offA, offB, acc);
  acc_settle();
  if (!busy) return;

  if (nsplit == 1) {
    // acc[a][b][v] = S(F0 + 128wa + 16a + 4g + v, G0 + 128wb + 64h + 16b + i16)
    const int g = lane >> 4;
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = F0 + 128 * wa + 16 * a + 4 * g + v;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t j = G0 + 128 * wb + 64 * h + 16 * b + i16;
          if (i < d && j < d && i <= j) {
            const float nv = S[i * d + j] + acc[a][b][v];
            S[i * d + j] = nv;
            if (i != j) S[j * d + i] = nv;
          }
        }
      }
  } else {
    // the 128x128 sub-tile's native accumulator order (column blocks
    // 4h .. 4h + 3 are this wave's): one contiguous 256-byte store per
    // (a, b, v)
    float* dst = part + ((int64_t(split) * ntiles + upper_index(ti, tj, nt)) * 4 + q) * kSubElems;
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          dst[((a * 8 + 4 * h + b) * 4 + v) * 64 + lane] = acc[a][b][v];
  }
}

// Adds the split partials of one 16 x 128 band (sub-tile wv, row block a) of
// an upper super-tile to S in split order (fp64 running sum), then mirrors
// the band into the lower triangle through LDS so both writes are row runs.
__global__ __launch_bounds__(256) void hessian_reduce_kernel(
    const float* __restrict__ part, int64_t d, int nt, int nsplit,
    float* __restrict__ S) {
  __shared__ float band[16][129];
  const int64_t L = blockIdx.x;
  const int wv = blockIdx.y >> 3, a = blockIdx.y & 7;
  int ti, tj;
  tile_of(L, nt, ti, tj);
  const bool diag = ti == tj;
  if (diag && wv == 2) return;
  const int wa = wv >> 1, wb = wv & 1;
  // thread t sums the eight consecutive partial values 8t .. 8t + 7 of the
  // band (accumulator register b8 * 4 + v, lanes l0 .. l0 + 7): eight
  // consecutive columns of one row
  const int tid = threadIdx.x;
  const int e0 = 8 * tid, bv = e0 >> 6, l0 = e0 & 63;
  const int row = 4 * (l0 >> 4) + (bv & 3);
  const int col0 = 16 * (bv >> 2) + (l0 & 15);
  const int64_t i0 = int64_t(ti) * kSup + 128 * wa + 16 * a;
  const int64_t j0 = int64_t(tj) * kSup + 128 * wb;
  const int64_t i = i0 + row;
  const int64_t ntiles = upper_tiles(nt);
  const float* src = part + (L * 4 + wv) * kSubElems + a * 8 * 4 * 64 + e0;
  const int64_t sstride = ntiles * 4 * kSubElems;
  // four splits per batch of 16-byte loads (the additions keep split order)
  double sum[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int s0 = 0; s0 < nsplit; s0 += 4) {
    f32x4 pv[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pv[u][h] = (s0 + u < nsplit)
                       ? *reinterpret_cast<const f32x4*>(src + (s0 + u) * sstride + 4 * h)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + u < nsplit) sum[k] += pv[u][k >> 2][k & 3];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int col = col0 + k;
    const int64_t j = j0 + col;
    float nv = 0.f;
    if (i < d && j < d && (!diag || i <= j)) {
      nv = static_cast<float>(static_cast<double>(S[i * d + j]) + sum[k]);
      S[i * d + j] = nv;
    }
    band[row][col] = nv;
  }
  __syncthreads();
  const int r = tid & 15;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int col = (tid >> 4) + 16 * k;
    const int64_t ii = i0 + r, jj = j0 + col;
    if (ii < d && jj < d && (!diag || ii < jj)) S[jj * d + ii] = band[r][col];
  }
}

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Generic path (fp32 activations, or bf16 rows that are not 16-byte
// aligned): 64x64 upper tiles, 4x4 outputs per thread, fp64 sums.
template <class T>
__global__ __launch_bounds__(256) void hessian_generic_kernel(
    const T* __restrict__ X, int64_t ldx, int64_t n_tok, int64_t d,
    int nt64, float* __restrict__ S) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  int ti, tj;
  tile_of(blockIdx.x, nt64, ti, tj);
  const int64_t F0 = int64_t(ti) * 64, G0 = int64_t(tj) * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4] = {};
  for (int64_t t0 = 0; t0 < n_tok; t0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int tt = e >> 6, ff = e & 63;
      const int64_t t = t0 + tt;
      As[tt][ff] = (t < n_tok && F0 + ff < d) ? to_f32(X[t * ldx + F0 + ff]) : 0.f;
      Bs[tt][ff] = (t < n_tok && G0 + ff < d) ? to_f32(X[t * ldx + G0 + ff]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = As[k][ty * 4 + u];
        bv[u] = Bs[k][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma(av[u], bv[w], acc[u][w]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int a = ty * 4 + u, b = tx * 4 + w;
      const int64_t i = F0 + a, j = G0 + b;
      if (i < d && j < d && (ti != tj || a <= b)) {
        const float nv = static_cast<float>(static_cast<double>(S[i * d + j]) + acc[u][w]);
        S[i * d + j] = nv;
        if (i != j) S[j * d + i] = nv;
      }
    }
}

struct SplitPlan {
  int nsplit;
  int64_t ks;
};

// Chooses the token split: (super-tile x split) work items run one workgroup
// per CU, so the MFMA time is (rounds of kCUs items) x (steps per split); the
// partial tiles cost a write and a read of 256 KiB per item.  Each split is
// one fp32 running sum per entry; splits of at most kMaxChain steps bound its
// rounding error (~steps * 2^-24 relative), as long as the partial tiles fit
// in max_part bytes.  Plans whose partial tiles exceed max_part are never
// chosen (one split needs none).
SplitPlan plan_splits(int64_t d, int64_t n_tok, double max_part) {
  const int64_t nt = (d + kSup - 1) / kSup;
  const int64_t ntiles = upper_tiles(nt);
  const int64_t steps = (n_tok + kStep - 1) / kStep;
  const double t_step = 1024.0 / 2.1e9;          // 64 MFMAs per SIMD per step
  const double t_byte = 1.0 / 4.0e12;
  SplitPlan best{1, steps * kStep};
  double best_t = 1e30;
  const int64_t max_split = std::min<int64_t>(64, steps);
  const double part_item = 4.0 * kSubElems * 4.0;
  int64_t min_split = 1;
  while (min_split < max_split && (steps + min_split - 1) / min_split > kMaxChain &&
         double(min_split + 1) * double(ntiles) * part_item <= max_part)
    ++min_split;
  for (int64_t ns = min_split; ns <= max_split; ++ns) {
    // an even step count per split keeps every split but the last on the
    // unmasked path
    const int64_t per = ((steps + ns - 1) / ns + 1) & ~int64_t(1);
    const int64_t nsr = (steps + per - 1) / per;
    if (nsr > 1 && double(nsr) * double(ntiles) * part_item > max_part) continue;
    const int64_t rounds = (ntiles * nsr + kCUs - 1) / kCUs;
    const double t = double(rounds) * double(per) * t_step +
                     (nsr > 1 ? 2.0 * double(nsr * ntiles) * 4.0 * kSubElems * 4.0 * t_byte : 0.0);
    if (t < best_t * 0.999) {
      best_t = t;
      best = SplitPlan{static_cast<int>(nsr), per * kStep};
    }
  }
  return best;
}

}  // namespace

size_t hessian_ws_bytes(int64_t d, int64_t n_tok, double max_part) {
  if (d <= 0 || n_tok <= 0) return 0;
  const SplitPlan p = plan_splits(d, n_tok, max_part);
  if (p.nsplit <= 1) return 0;
  const int64_t nt = (d + kSup - 1) / kSup;
  return align_up(size_t(p.nsplit) * size_t(upper_tiles(nt)) * 4 * kSubElems * sizeof(float));
}

namespace {
bool mfma_path_ok(int64_t d, const void* X, gptq_dtype dt, int64_t ldx) {
  // per-lane byte offsets of a 32-token step are kept in 32 bits
  return dt == GPTQ_BF16 && d % 8 == 0 && ldx % 8 == 0 &&
         reinterpret_cast<uintptr_t>(X) % 16 == 0 &&
         2 * (int64_t(kStep) * ldx + d) < (int64_t(1) << 32);
}
}  // namespace

gptq_status launch_hessian(float* S, int64_t d, const void* X, gptq_dtype dt,
                           int64_t n_tok, int64_t ldx, void* ws,
                           hipStream_t st, double max_part) {
  if (n_tok == 0) return GPTQ_OK;
  if (!mfma_path_ok(d, X, dt, ldx)) {
    const int nt64 = static_cast<int>((d + 63) / 64);
    const dim3 grid(static_cast<unsigned>(upper_tiles(nt64)));
    if (dt == GPTQ_F32)
      hessian_generic_kernel<float><<<grid, 256, 0, st>>>(
          static_cast<const float*>(X), ldx, n_tok, d, nt64, S);
    else
      hessian_generic_kernel<uint16_t><<<grid, 256, 0, st>>>(
          static_cast<const uint16_t*>(X), ldx, n_tok, d, nt64, S);
    GPTQ_CHECK_LAUNCH();
    return GPTQ_OK;
  }
  const int nt = static_cast<int>((d + kSup - 1) / kSup);
  const SplitPlan p = plan_splits(d, n_tok, max_part);
  const int64_t nitems = upper_tiles(nt) * p.nsplit;
  const dim3 grid(static_cast<unsigned>((nitems + kCUs - 1) / kCUs * kCUs));
  hessian_bf16_kernel<true><<<grid, kThreads, 0, st>>>(
      static_cast<const uint16_t*>(X), ldx, n_tok, d, nt, p.ks, p.nsplit, S,
      static_cast<float*>(ws));
  GPTQ_CHECK_LAUNCH();
  // masked items: panels crossing d, or a last split that is not a whole
  // number of 32-token steps (every other split is, see plan_splits)
  const int64_t last = n_tok - int64_t(p.nsplit - 1) * p.ks;
  if (d % kSup != 0 || last % kStep != 0) {
    hessian_bf16_kernel<false><<<grid, kThreads, 0, st>>>(
        static_cast<const uint16_t*>(X), ldx, n_tok, d, nt, p.ks, p.nsplit, S,
        static_cast<float*>(ws));
    GPTQ_CHECK_LAUNCH();
  }
  if (p.nsplit > 1) {
    hessian_reduce_kernel<<<dim3(static_cast<unsigned>(upper_tiles(nt)), 32), 256, 0, st>>>(
        static_cast<const float*>(ws), d, nt, p.nsplit, S);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}

}  // namespace gptq
