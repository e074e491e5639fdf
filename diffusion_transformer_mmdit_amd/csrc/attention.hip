// Joint multi-head attention O = softmax(Q K^T / sqrt(128)) V over the whole [txt ; img]
// sequence, no mask (the scaled dot-product attention formula of the kwkr.cn article,
// section 2; "Joint multi-head attention: separate QKV, shared attention" of the Klein 9B
// shape trace, section 4).
//
// bf16 path (gfx950 MFMA 32x32x16, fp32 softmax and accumulation), flash style:
//   * a workgroup of NW waves owns 32*NW queries of one (batch, head); each wave keeps
//     the Q fragments of its 32 queries in registers for the whole key loop;
//   * K tiles [64 keys][128] and V^T tiles [128][64 keys] are staged in LDS by direct
//     global->LDS loads, double buffered.  V arrives already transposed (V^T, written by
//     the QKV projection's epilogue), so no transposition happens here;
//   * scores are computed transposed, S^T = K Q^T, so each lane owns one query and 32 of
//     the tile's 64 keys; the K rows are fed to the MFMA in a permuted order chosen so
//     that every lane's 8 probabilities of a 16-key chunk are 8 CONSECUTIVE keys, which
//     makes the V^T fragment of O^T = V^T P^T a single 16-byte LDS read;
//   * softmax in the exp2 domain (log2(e)/sqrt(d) folded into one FMA per score).  Each
//     row takes the maximum of its first key tile and keeps it: later tiles take no
//     maximum at all.  Any later score up to ~2^7 above it leaves p and the fp32 row sum
//     finite, and nothing below it is lost (the first tile's best key alone gives a row
//     sum >= 1), so the result is the same softmax.  If some row's sum or output is not
//     finite after the loop, the workgroup recomputes its key range with a lazy running
//     maximum (O and the sum rescaled only when a row's maximum grows by more than 2^8).
//     Row sums are fp32 adds of the unrounded probabilities, P enters the PV product in
//     bf16;
//   * the key loop is software pipelined: while a wave takes the exponentials of one tile
//     it already computes the next tile's scores, so its own MFMAs run beside its softmax
//     (K is loaded two tiles ahead, V one tile ahead, one barrier per tile);
//   * two workgroups per CU (<= 256 registers per wave) so one workgroup's softmax
//     overlaps the other's MFMAs;
//   * work units are (query block, head, batch).  Units that fill whole rounds of resident
//     workgroups run whole; each unit of a partial last round is split along the keys into
//     `splits` ranges whose unnormalised fp32 partial outputs, running maxima and sums a
//     second kernel merges in a fixed order (the usual rescale-and-sum of flash-attention
//     partials), so the last round is not left mostly idle.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace flux {

template <class T>
FLUX_DEV const T* seq_cptr(const SeqView& v, int b, int j) {
  return (j < v.n0) ? static_cast<const T*>(v.base0) + b * v.bs0 + (int64_t)j * v.ld
                    : static_cast<const T*>(v.base1) + b * v.bs1 + (int64_t)(j - v.n0) * v.ld;
}
template <class T>
FLUX_DEV T* seq_mptr(const SeqView& v, int b, int j) {
  return (j < v.n0) ? static_cast<T*>(v.base0) + b * v.bs0 + (int64_t)j * v.ld
                    : static_cast<T*>(v.base1) + b * v.bs1 + (int64_t)(j - v.n0) * v.ld;
}

constexpr int kHD = 128;   // head dim
constexpr int kBKV = 64;   // keys per tile

// K tile: 64 rows of 256 B (16 chunks); chunk c of row r sits at slot c ^ (r & 15)
FLUX_DEV int k_off(int row, int c) { return row * kHD + ((c ^ (row & 15)) << 3); }
// V^T tile: 128 rows (d) of 128 B (8 chunks of 8 keys); slot = c ^ ((d >> 1) & 7)
FLUX_DEV int v_off(int d, int c) { return d * kBKV + ((c ^ ((d >> 1) & 7)) << 3); }
// MFMA row m of a 32-key S^T block reads key sigma(m) of the block: with
// m = 8q + 4g + t the lane group g of register block q gets keys 16(q>>1) + 8g + 4(q&1) + t
FLUX_DEV int key_perm(int m) {
  const int q = m >> 3, g = (m >> 2) & 1, t = m & 3;
  return 16 * (q >> 1) + 8 * g + 4 * (q & 1) + t;
}

// Direct loads with operands forced into scalar registers (readfirstlane; a no-op for
// values the compiler already holds there).  The extra-key variant of the kernel uses them:
// with its second key source the compiler no longer proves these operands uniform itself.
FLUX_DEV const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
template <bool U>
FLUX_DEV void dma_s(const void* base, uint32_t voff, uint32_t lds) {
  if constexpr (U)
    dma16s(uniform_ptr(base), voff, __builtin_amdgcn_readfirstlane(lds));
  else
    dma16s(base, voff, lds);
}
template <bool U>
FLUX_DEV void dma_v(const void* g, uint32_t lds) {
  if constexpr (U)
    dma16v(g, __builtin_amdgcn_readfirstlane(lds));
  else
    dma16v(g, lds);
}

// Unit u = (b * heads + head) * nqb + qb (query blocks of one head are consecutive, so a
// run of units on one XCD shares that head's K and V in L2).
FLUX_DEV int attn_xcd_remap(int bid, int total) {
  return ((total & 7) == 0) ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
}

// EXTRA: key tiles past the sequence's own come from the extra source `xkv` (see KvExtra).
// The 64 KB of LDS per workgroup allow 2 workgroups per CU: 2 waves per SIMD with 4-wave
// workgroups (so at most 256 registers each), 1 with 2-wave ones (which may use AGPRs).
template <int NW, bool EXTRA>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void flash_attn_bf16_kernel(
    SeqView qv, SeqView kv, const bf16* __restrict__ vt, int64_t ld_vt, int dim, SeqView ov,
    int seq, float scale_log2, int nqb, int heads, int full_units, int splits,
    float* __restrict__ partial, KvExtra xkv, int o_f16) {
  constexpr int NT = 64 * NW;
  __shared__ __align__(16) bf16 Ks[2][kBKV * kHD];
  __shared__ __align__(16) bf16 Vs[2][kHD * kBKV];

  const int nm = (seq + kBKV - 1) / kBKV;  // tiles of the sequence's own keys
  const int ntiles = nm + (EXTRA ? (xkv.n + kBKV - 1) / kBKV : 0);
  int unit, t_begin = 0, t_end = ntiles, part = -1;
  if ((int)blockIdx.x < full_units) {
    unit = attn_xcd_remap(blockIdx.x, full_units);
  } else {
    part = blockIdx.x - full_units;
    unit = full_units + part / splits;
    const int sp = part % splits;
    t_begin = sp * ntiles / splits;
    t_end = (sp + 1) * ntiles / splits;
  }
  const int qb = unit % nqb;
  const int head = (unit / nqb) % heads, b = unit / (nqb * heads);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int q0 = qb * (32 * NW) + wave * 32;
  const int hoff = head * kHD;

  // ---- Q fragments (B operand of S^T = K Q^T): query l32, dims 16 kk + 8 g .. + 8
  bf16x8 qf[8];
  {
    const int qi = min(q0 + l32, seq - 1);
    const bf16* qp = seq_cptr<bf16>(qv, b, qi) + hoff + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    // compiler-visible vmcnt(0): the compiler does not count the asm K/V loads, so a wait
    // it derived for these Q loads inside the key loop would also stall on those
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // ---- direct-load plan.  K: one wave instruction = 4 rows x 256 B; lane -> row
  // (lane >> 4), slot (lane & 15).  V^T: one instruction = 8 rows x 128 B; lane -> row
  // (lane >> 3), slot (lane & 7).  Each lane fetches the logical chunk of its slot.  A key
  // tile that lies inside one segment of the key view and inside the sequence is addressed
  // as a scalar base (per tile) + a fixed per-lane byte offset, so issuing it costs no
  // vector instructions; other tiles (the last one, one straddling the txt/img boundary)
  // take per-lane addresses with the key clamped to the sequence.
  constexpr int KI = 16 / NW;  // K instructions per wave per tile (64 rows / 4)
  constexpr int VI = 16 / NW;  // V instructions per wave per tile (128 rows / 8)
  const bf16* vt_head = vt + ((int64_t)b * dim + hoff) * ld_vt;
  // per-lane byte offsets of load j of a K tile (row stride ld) and a V^T tile (ld_v)
  auto k_lane_off = [&](int j, int64_t ld) __attribute__((always_inline)) {
    const int row = (wave * KI + j) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    return (uint32_t)(((int64_t)row * ld + hoff + c * 8) * 2);
  };
  auto v_lane_off = [&](int j, int64_t ld_v) __attribute__((always_inline)) {
    const int d = (wave * VI + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((d >> 1) & 7);
    return (uint32_t)(((int64_t)d * ld_v + c * 8) * 2);
  };
  // recomputed per tile (a few VALU operations) rather than held in registers: the
  // pipelined key loop keeps two tiles' scores live
  auto kvo = [&](int j) __attribute__((always_inline)) { return k_lane_off(j, kv.ld); };
  auto vvo = [&](int j) __attribute__((always_inline)) { return v_lane_off(j, ld_vt); };
  const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ks0 = __builtin_amdgcn_readfirstlane(lds_u32(&Ks[0][0])) + wv * KI * 4 * kHD * 2;
  const uint32_t vs0 = __builtin_amdgcn_readfirstlane(lds_u32(&Vs[0][0])) + wv * VI * 8 * kBKV * 2;
  constexpr uint32_t KBUF = kBKV * kHD * 2, VBUF = kHD * kBKV * 2;
  // tile of the extra source at key x0: scalar base + per-lane offsets while the tile lies
  // inside the extra keys, else per-lane addresses with the key clamped to the last one.
  // The extra source's fields are read into scalars once (a by-reference capture of the
  // argument struct would place it in per-lane memory).
  const bf16* xk = nullptr;
  const bf16* xvt = nullptr;
  int64_t xld = 0, xldv = 0;
  int xn = 0;
  if constexpr (EXTRA) {
    const int bx = b % xkv.nb;
    xk = static_cast<const bf16*>(xkv.k) + bx * xkv.bs;
    xvt = static_cast<const bf16*>(xkv.vt) + ((int64_t)bx * dim + hoff) * xkv.ld_vt;
    xld = xkv.ld;
    xldv = xkv.ld_vt;
    xn = xkv.n;
  }
  // K rows of key tile `it` into K buffer `buf`.  A tile inside one segment of its key
  // source takes the scalar base + per-lane offsets; others (the last one, one straddling
  // the txt/img boundary) per-lane addresses with the key clamped to the source's last.
  auto issue_k = [&](int buf, int it) __attribute__((always_inline)) {
    const uint32_t dst = ks0 + buf * KBUF;
    if constexpr (EXTRA) {
      if (it >= nm) {
        const int x0 = (it - nm) * kBKV;
        if (x0 + kBKV <= xn) {
          const bf16* kb = xk + (int64_t)x0 * xld;
#pragma unroll
          for (int j = 0; j < KI; ++j) dma_s<true>(kb, k_lane_off(j, xld), dst + j * 4 * kHD * 2);
        } else {
#pragma unroll
          for (int j = 0; j < KI; ++j) {
            const int row = (wave * KI + j) * 4 + (lane >> 4);
            const int key = min(x0 + row, xn - 1);
            const int c = (lane & 15) ^ (row & 15);
            dma_v<true>(xk + (int64_t)key * xld + hoff + c * 8, dst + j * 4 * kHD * 2);
          }
        }
        return;
      }
    }
    const int kv0 = it * kBKV;
    const bool in0 = kv0 + kBKV <= kv.n0, in1 = kv0 >= kv.n0;
    if ((in0 || in1) && kv0 + kBKV <= seq) {
      const bf16* kb = in0 ? static_cast<const bf16*>(kv.base0) + b * kv.bs0 + (int64_t)kv0 * kv.ld
                           : static_cast<const bf16*>(kv.base1) + b * kv.bs1 +
                                 (int64_t)(kv0 - kv.n0) * kv.ld;
#pragma unroll
      for (int j = 0; j < KI; ++j) dma_s<EXTRA>(kb, kvo(j), dst + j * 4 * kHD * 2);
    } else {
#pragma unroll
      for (int j = 0; j < KI; ++j) {
        const int row = (wave * KI + j) * 4 + (lane >> 4);
        const int key = min(kv0 + row, seq - 1);  // past the end: a valid row, masked later
        const int c = (lane & 15) ^ (row & 15);
        dma_v<EXTRA>(seq_cptr<bf16>(kv, b, key) + hoff + c * 8, dst + j * 4 * kHD * 2);
      }
    }
  };
  // V^T columns of key tile `it` into V buffer `buf` (the V^T rows are padded to whole
  // tiles, so a partial tile reads padding, never past the rows)
  auto issue_v = [&](int buf, int it) __attribute__((always_inline)) {
    const uint32_t dst = vs0 + buf * VBUF;
    if constexpr (EXTRA) {
      if (it >= nm) {
        const int x0 = (it - nm) * kBKV;
#pragma unroll
        for (int j = 0; j < VI; ++j) dma_s<true>(xvt + x0, v_lane_off(j, xldv), dst + j * 8 * kBKV * 2);
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < VI; ++j) dma_s<EXTRA>(vt_head + it * kBKV, vvo(j), dst + j * 8 * kBKV * 2);
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int krow0 = key_perm(l32), krow1 = 32 + key_perm(l32);

  // per-lane LDS element offsets of the fragments: K rows krow0 (krow1 = krow0 + 32 has
  // the same swizzle, so its fragments sit 32 rows further) for each of the 8 k-steps;
  // V^T rows 32 dt + l32 (the swizzle depends only on l32) for each 16-key chunk c
  int koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = k_off(krow0, 2 * kk + g);
#pragma unroll
  for (int c = 0; c < 4; ++c) voff[c] = v_off(l32, 2 * c + g);

  // S^T = K Q^T of the key tile in K buffer BUF: s[h] covers MFMA rows of key block h
  // (keys 32 h + key_perm(row)); register r of block h holds key 32 h + 16 (r >> 3) +
  // 8 g + (r & 7)
  auto scores = [&](f32x16 (&s)[2], auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[h][r] = 0.f;
    // K fragments read one k-step ahead of their MFMAs
    bf16x8 ka[2], kb[2];
    ka[0] = *reinterpret_cast<const bf16x8*>(&Ks[buf][koff[0]]);
    kb[0] = *reinterpret_cast<const bf16x8*>(&Ks[buf][koff[0] + 32 * kHD]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (kk + 1 < 8) {
        ka[(kk + 1) & 1] = *reinterpret_cast<const bf16x8*>(&Ks[buf][koff[kk + 1]]);
        kb[(kk + 1) & 1] = *reinterpret_cast<const bf16x8*>(&Ks[buf][koff[kk + 1] + 32 * kHD]);
      }
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk & 1], qf[kk], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[kk & 1], qf[kk], s[1], 0, 0, 0);
    }
  };

  // One key tile, software pipelined with the next one so that a wave's softmax (VALU)
  // runs beside MFMAs of its own instead of alternating with them.  Tile t of the range
  // lives in LDS buffers (t - t_begin) & 1 = CUR.  On entry the tile's scores are in sc,
  // its V^T in V buffer CUR and the next tile's K in K buffer CUR ^ 1.  The step refills
  // K buffer CUR with tile it + 2 and V buffer CUR ^ 1 with tile it + 1, computes the next
  // tile's scores into sn (NEXT) between this tile's exponentials, and adds V^T P^T to O.
  // FIXED: the row maximum of an earlier tile stands (no maximum is taken).
  auto step = [&](int it, auto cur_c, auto next_c, f32x16 (&sc)[2], f32x16 (&sn)[2],
                  auto fixed_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr bool FIXED = decltype(fixed_c)::value;
    // a tile reaching past its source's keys (`lim` of them in the tile) is masked
    const int lim = (EXTRA && it >= nm) ? xn - (it - nm) * kBKV : seq - it * kBKV;
    if (lim < kBKV) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * h + 16 * (r >> 3) + 8 * g + (r & 7) >= lim) sc[h][r] = -INFINITY;
    }
    if constexpr (!FIXED) {
      // online softmax in the log2 domain with a lazily updated maximum: O and the sum are
      // rescaled only when some row's maximum grows by more than 2^8 (every row on the first
      // tile, rarely afterwards), so p <= 256
      float mx4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) mx4[i] = fmaxf(sc[0][i], sc[1][i]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 4 * (1 - h); r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], sc[h][r]);
      float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
      {
        // lane l and lane l ^ 32 hold the two halves of one query's keys: exchange the
        // halves in registers (v_permlane32_swap) instead of through LDS
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
      }
      const bool grow = mx > m_run + 8.f;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m_run = m_new;
      }
    }
    if (it + 2 < t_end) issue_k(cur, it + 2);
    if (NEXT) issue_v(cur ^ 1, it + 1);

    if constexpr (NEXT) scores(sn, std::integral_constant<int, cur ^ 1>{});
    // raw v_exp_f32: arguments are <= 8 with the lazy maximum (with a kept one they stay
    // finite unless the overflow check after the loop fires); results below 2^-126 may
    // flush to zero
    float p[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[h][r] = __builtin_amdgcn_exp2f(fmaf(sc[h][r], scale_log2, -m_run));
    // the row sum in fp32 over the unrounded probabilities (plain adds run beside the
    // MFMAs; bf16 dot products against (1, 1) would take the matrix pipe's turn), P in
    // bf16 as the PV product's operand
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) ls[r & 3] += p[h][r];
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    uint32_t pw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pw[i] = pack2(p[i >> 3][2 * (i & 7)], p[i >> 3][2 * (i & 7) + 1]);

    // O^T += V^T P^T over 4 chunks of 16 keys; lane group g owns keys 16 c + 8 g .. + 8
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&Vs[cur][voff[c] + 32 * dt * kBKV]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[dt], 0, 0, 0);
      }
    }

    // this wave's refills landed; after the barrier every wave's have, and every wave is
    // done reading the buffers the next step refills
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;
  using On = std::true_type;
  using Off = std::false_type;
  // The key loop.  The first tile always takes the row maximum (m_run starts at -inf, so
  // every row adopts its first tile's maximum).  FIXED_REST: the later tiles keep that
  // maximum and take none of their own; the result stands unless some score exceeded it by
  // enough to overflow the fp32 sum, which the caller checks afterwards.
  auto key_loop = [&](auto fixed_rest) __attribute__((always_inline)) {
    using Rest = decltype(fixed_rest);
    issue_k(0, t_begin);
    issue_v(0, t_begin);
    if (t_begin + 1 < t_end) issue_k(1, t_begin + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sa[2], sb[2];
    scores(sa, Buf0{});
    __syncthreads();  // K buffer 0 is refilled by the first step
    int it = t_begin;
    if (it + 1 < t_end) {
      step(it++, Buf0{}, On{}, sa, sb, Off{});
      for (; it + 2 < t_end; it += 2) {
        step(it, Buf1{}, On{}, sb, sa, Rest{});
        step(it + 1, Buf0{}, On{}, sa, sb, Rest{});
      }
      if (it + 1 < t_end) {
        step(it, Buf1{}, On{}, sb, sa, Rest{});
        step(it + 1, Buf0{}, Off{}, sa, sb, Rest{});
      } else {
        step(it, Buf1{}, Off{}, sb, sa, Rest{});
      }
    } else {
      step(it, Buf0{}, Off{}, sa, sb, Off{});
    }
  };
  if (t_begin < t_end) {
    key_loop(On{});
    // With the first tile's maximum m kept, p = 2^(s - m) stays finite unless a later score
    // exceeds m by ~2^7; then the row sum or O is no longer finite.  (Below m nothing is
    // lost: the first tile's best key alone gives a row sum >= 1.)  If any row of the
    // workgroup overflowed, the whole range is recomputed with the lazily updated maximum.
    float osum = l_run;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) osum += o[dt][r];
    if (__syncthreads_or(!__builtin_isfinite(osum))) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
      m_run = -INFINITY;
      l_run = 0.f;
      key_loop(Off{});
    }
  }

  // lane owns query l32 and dims 32 dt + 8 (r/4) + 4 g + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int qi = q0 + l32;
  if (part >= 0) {
    // split unit: unnormalised O, running maximum (log2 domain) and sum for the merge
    const int ql = wave * 32 + l32;
    float* op = partial + ((int64_t)part * NT / 2 + ql) * kHD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(op + 32 * dt + 8 * r4 + 4 * g) =
            make_float4(o[dt][4 * r4], o[dt][4 * r4 + 1], o[dt][4 * r4 + 2], o[dt][4 * r4 + 3]);
    if (g == 0) {
      // (maximum, sum) pairs follow the O rows of all split units
      const int n_parts = gridDim.x - full_units;
      float* ml = partial + (int64_t)n_parts * (NT / 2) * kHD + ((int64_t)part * NT / 2 + ql) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
    return;
  }
  // normalise and write O[query][d] (bf16, or binary16 with o_f16)
  const float inv = 1.f / l_tot;
  if (qi < seq) {
    bf16* op = seq_mptr<bf16>(ov, b, qi) + hoff;
    auto put = [&](auto pk2) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * dt + 8 * r4 + 4 * g;
          *reinterpret_cast<uint2*>(op + d) =
              make_uint2(pk2(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv),
                         pk2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv));
        }
    };
    if (o_f16)
      put([](float x, float y) { return pack2h(x, y); });
    else
      put([](float x, float y) { return pack2(x, y); });
  }
}

// Merge of the split units: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s, splits taken in order.  One thread per (query, 4 dims); grid.x walks the
// split units' queries, QPU = queries per unit.
template <int QPU>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ partial,
                                                         int64_t ml_offset, int splits,
                                                         int n_units, int full_units, int nqb,
                                                         int heads, int seq, SeqView ov,
                                                         int o_f16) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d4 = (int)(idx & 31);
  const int64_t uq = idx >> 5;  // split unit * QPU + query
  if (uq >= (int64_t)n_units * QPU) return;
  const int tu = (int)(uq / QPU), ql = (int)(uq % QPU);
  const int unit = full_units + tu;
  const int qb = unit % nqb, head = (unit / nqb) % heads, b = unit / (nqb * heads);
  const int qi = qb * QPU + ql;
  if (qi >= seq) return;
  const float* ml = partial + ml_offset;
  float mmax = -INFINITY;
  for (int sp = 0; sp < splits; ++sp)
    mmax = fmaxf(mmax, ml[(((int64_t)tu * splits + sp) * QPU + ql) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t row = ((int64_t)tu * splits + sp) * QPU + ql;
    const float w = exp2f(ml[row * 2] - mmax);
    lsum += w * ml[row * 2 + 1];
    const float4 v = *reinterpret_cast<const float4*>(partial + row * kHD + 4 * d4);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = 1.f / lsum;
  bf16* op = seq_mptr<bf16>(ov, b, qi) + head * kHD + 4 * d4;
  *reinterpret_cast<uint2*>(op) =
      o_f16 ? make_uint2(pack2h(acc.x * inv, acc.y * inv), pack2h(acc.z * inv, acc.w * inv))
            : make_uint2(pack2(acc.x * inv, acc.y * inv), pack2(acc.z * inv, acc.w * inv));
}

// fp32 path (tiny fp32 workloads): one wave per (query, head); each lane owns 2 dims.
__global__ __launch_bounds__(64) void attn_f32_kernel(SeqView qv, SeqView kv,
                                                      const float* __restrict__ vt, int64_t ld_vt,
                                                      int dim, SeqView ov, int seq, float scale,
                                                      KvExtra xkv) {
  const int lane = threadIdx.x;
  const int qi = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int d = head * kHD + 2 * lane;
  const float* qp = seq_cptr<float>(qv, b, qi) + d;
  const float q0 = qp[0], q1 = qp[1];
  const float* v0 = vt + ((int64_t)b * dim + d) * ld_vt;
  const float* v1 = v0 + ld_vt;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < seq; ++j) {
    const float* kp = seq_cptr<float>(kv, b, j) + d;
    const float s = wave_sum(q0 * kp[0] + q1 * kp[1]) * scale;
    const float m_new = fmaxf(m, s);
    const float a = expf(m - m_new), p = expf(s - m_new);
    l = l * a + p;
    o0 = o0 * a + p * v0[j];
    o1 = o1 * a + p * v1[j];
    m = m_new;
  }
  if (xkv.n > 0) {
    const int bx = b % xkv.nb;
    const float* xk = static_cast<const float*>(xkv.k) + bx * xkv.bs + d;
    const float* xv0 = static_cast<const float*>(xkv.vt) + ((int64_t)bx * dim + d) * xkv.ld_vt;
    const float* xv1 = xv0 + xkv.ld_vt;
    for (int j = 0; j < xkv.n; ++j) {
      const float* kp = xk + (int64_t)j * xkv.ld;
      const float s = wave_sum(q0 * kp[0] + q1 * kp[1]) * scale;
      const float m_new = fmaxf(m, s);
      const float a = expf(m - m_new), p = expf(s - m_new);
      l = l * a + p;
      o0 = o0 * a + p * xv0[j];
      o1 = o1 * a + p * xv1[j];
      m = m_new;
    }
  }
  float* op = seq_mptr<float>(ov, b, qi) + d;
  op[0] = o0 / l;
  op[1] = o1 / l;
}

static int attn_waves(int seq, int heads, int batch) {
  // 64 KB of LDS per workgroup limits a CU to 2 resident workgroups.  4-wave workgroups
  // (2 waves per SIMD) unless there are fewer of them than CUs: measured on MI355X, they
  // are 15-28% faster from 288 to 480 units (L 1536-2560 with 24 heads) and equal or
  // slower below 256 (L 640: 21.6 vs 21.4 us; L 1024: 34.9 vs 31.4 us).
  const int cus = 256;
  const long wg4 = (long)((seq + 127) / 128) * heads * batch;
  return wg4 >= cus ? 4 : 2;
}

// Largest partial-output footprint: at most one round of resident workgroups (2 per CU)
// of split units, 128 queries each, 128 dims + (maximum, sum) per query.
constexpr int kAttnSlots = 2 * 256;
size_t attention_split_bytes() { return (size_t)kAttnSlots * 128 * (kHD + 2) * sizeof(float); }

template <int NW, bool EXTRA>
static hipError_t launch_flash(SeqView q, SeqView k, const bf16* vt, int64_t ld_vt, int dim,
                               SeqView o, int batch, int seq, int heads, float* split_ws,
                               const KvExtra& x, int o_f16, hipStream_t s) {
  constexpr int QPU = 32 * NW;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHD);
  const int nqb = (seq + QPU - 1) / QPU;
  const int units = nqb * heads * batch;
  const int ntiles = (seq + kBKV - 1) / kBKV + (EXTRA ? (x.n + kBKV - 1) / kBKV : 0);
  // split the partial last round along the keys (at least 4 key tiles per range)
  int tail = units % kAttnSlots, splits = 1;
  if (split_ws != nullptr && tail > 0 && 2 * tail <= kAttnSlots) {
    splits = kAttnSlots / tail;
    if (splits > ntiles / 4) splits = ntiles / 4;
  } else if (split_ws != nullptr && units > 256 && units < kAttnSlots && units - 256 <= 128) {
    // fewer units than resident slots but more than CUs: one whole unit per CU, the rest
    // split along the keys beside them (L 1536 x 24 heads, 288 units: 56.2 -> 53.6 us
    // against 32 CUs running two whole units)
    tail = units - 256;
    splits = 256 / tail;
    if (splits > ntiles / 4) splits = ntiles / 4;
  }
  if (splits < 2) {
    splits = 1;
    tail = 0;
  }
  const int full = units - tail;
  const int grid = full + tail * splits;
  hipLaunchKernelGGL((flash_attn_bf16_kernel<NW, EXTRA>), dim3(grid), dim3(64 * NW), 0, s, q, k, vt,
                     ld_vt, dim, o, seq, scale_log2, nqb, heads, full, splits, split_ws, x,
                     o_f16);
  if (tail > 0) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ml_offset = (int64_t)tail * splits * QPU * kHD;  // after the split units' O rows
    const int64_t threads = (int64_t)tail * QPU * 32;
    hipLaunchKernelGGL(attn_merge_kernel<QPU>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, split_ws, ml_offset, splits, tail, full, nqb, heads, seq, o, o_f16);
  }
  return hipGetLastError();
}

hipError_t attention(int dtype, SeqView q, SeqView k, const void* vt, int64_t ld_vt, SeqView o,
                     int batch, int seq, int heads, float* split_ws, hipStream_t s,
                     const KvExtra* extra, int o_dtype) {
  if (seq <= 0 || batch <= 0) return hipSuccess;
  const int dim = heads * kHD;
  KvExtra x{};
  x.nb = 1;
  if (extra != nullptr && extra->n > 0) x = *extra;
  if (dtype == DT_BF16) {
    if (o_dtype < 0) o_dtype = DT_BF16;
    if (o_dtype != DT_BF16 && o_dtype != DT_F16) return hipErrorInvalidValue;
    const int of16 = o_dtype == DT_F16;
    const bf16* v = static_cast<const bf16*>(vt);
    // extra keys: 4-wave workgroups only (the 2-wave variant of the extra-source path does
    // not fit the register budget)
    if (x.n > 0)
      return launch_flash<4, true>(q, k, v, ld_vt, dim, o, batch, seq, heads, split_ws, x, of16, s);
    if (attn_waves(seq, heads, batch) == 4)
      return launch_flash<4, false>(q, k, v, ld_vt, dim, o, batch, seq, heads, split_ws, x, of16,
                                    s);
    return launch_flash<2, false>(q, k, v, ld_vt, dim, o, batch, seq, heads, split_ws, x, of16, s);
  } else {
    dim3 grid(seq, heads, batch);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), 0, s, q, k, static_cast<const float*>(vt),
                       ld_vt, dim, o, seq, 1.f / sqrtf((float)kHD), x);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// V -> V^T (for callers that hold V token-major) and zeroing of the V^T row padding
// ------------------------------------------------------------------------------------
template <class T>
__global__ void transpose_v_kernel(SeqView v, T* __restrict__ vt, int64_t ld_vt, int dim,
                                   int seq) {
  __shared__ T tile[32][33];
  const int b = blockIdx.z;
  const int j0 = blockIdx.x * 32, f0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8 threads
  for (int r = ty; r < 32; r += 8) {
    const int j = j0 + r, f = f0 + tx;
    tile[r][tx] = (j < seq && f < dim) ? seq_cptr<T>(v, b, j)[f] : T(0.f);
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int f = f0 + r, j = j0 + tx;
    if (f < dim && j < seq) vt[((int64_t)b * dim + f) * ld_vt + j] = tile[tx][r];
  }
}

hipError_t transpose_v(int dtype, SeqView v, void* vt, int64_t ld_vt, int dim, int batch, int seq,
                       hipStream_t s) {
  dim3 grid((seq + 31) / 32, (dim + 31) / 32, batch), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(transpose_v_kernel<bf16>, grid, block, 0, s, v, static_cast<bf16*>(vt),
                       ld_vt, dim, seq);
  else
    hipLaunchKernelGGL(transpose_v_kernel<float>, grid, block, 0, s, v, static_cast<float*>(vt),
                       ld_vt, dim, seq);
  return hipGetLastError();
}

template <class T>
__global__ void zero_cols_kernel(T* __restrict__ p, int64_t ld, int64_t rows, int c0, int c1) {
  const int w = c1 - c0;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * w) return;
  const int64_t r = idx / w;
  p[r * ld + c0 + (idx % w)] = T(0.f);
}

hipError_t zero_cols(int dtype, void* p, int64_t ld, int64_t rows, int c0, int c1, hipStream_t s) {
  const int64_t total = rows * (c1 - c0);
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(zero_cols_kernel<bf16>, grid, block, 0, s, static_cast<bf16*>(p), ld, rows,
                       c0, c1);
  else
    hipLaunchKernelGGL(zero_cols_kernel<float>, grid, block, 0, s, static_cast<float*>(p), ld, rows,
                       c0, c1);
  return hipGetLastError();
}

}  // namespace flux
