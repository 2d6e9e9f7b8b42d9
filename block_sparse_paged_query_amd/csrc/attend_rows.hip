// Block-sparse decode attend over a paged KV cache: one query row (of a
// request's decode_query_len rows) per workgroup and kv head.
//
// [FI] vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
//      MiniMaxM3SparseFlashInferImpl.forward: GQA decode over the selected
//      blocks, causal, right-aligned positions, fp8 scales folded into the
//      softmax scale and the output.
// [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4,
//      MiniMaxM3SparseRocmNvfp4Impl / customize_spec: NVFP4 pages, two head
//      slots (K, V) per kv head.
// [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa,
//      _write_sparse_block_table_row_from_values: which tokens a row sees.
//
// Work decomposition.  A unit (row, kv head, split) is served by W = 3 or 4
// waves, chosen at launch so that the grid fills whole rounds of the
// machine; a workgroup holds one unit, or four 3-wave units when they fill
// the machine once (see attend_rows_kernel).  The unit's first wave compacts
// the row's top-k ids into the slot list (full blocks, then the causal tail)
// in LDS.  The row's context [0, ctx) is cut into 32-token chunks (two
// 16-token pages of one 128-token block); a split owns a contiguous range of
// chunks and its W waves take every W-th chunk.  Each wave keeps its own
// online-softmax state and several chunks' loads in flight; the W states are
// merged through LDS at the end.  With one split the unit writes the bf16
// output directly; otherwise it writes an fp32 partial (o, m, l) and
// attend_merge combines.
//
// Loads go through raw-buffer descriptors built per page in scalar
// registers, sized to the page's tokens inside the context: the hardware
// returns 0 for the rest, so neither the tail nor a bad block id needs a
// branch or a select per load, and lane addresses are loop constants.
//
// Per chunk, one wave computes S^T = K Q^T (tokens x heads) and
// O^T += V^T P^T (head_dim x heads) on 16x16x32 matrix cores, the GQA group
// padded to 16 heads.  Lane l = 16g + r:
//   K operand: token r of page 0 (tile 0) / page 1 (tile 1), d = kappa(kk,g,e)
//   S output:  tokens 4g+i (tile 0) and 16+4g+i (tile 1), head r
//   P operand: exactly those 8 probabilities, so the reduction index k of
//              the PV product is the chunk token tau(8g+i) = 4g+i (i<4),
//              16+4g+i-4 (i>=4)
//   V operand: rows tau(8g+0..7), columns d = r*NN + nn (NN = D/16): each
//              lane loads 8 token rows of NN consecutive elements and
//              transposes them in registers (no LDS round trip)
//   O output:  head r, d = (4g+i)*NN + nn, i.e. 4*NN consecutive d per lane.
#include <algorithm>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

// d index of element e of the K / Q operand for reduction step kk, lane group
// g: chosen so that each lane's loads are 16 contiguous bytes and a quarter
// wave covers contiguous runs of a token row.
template <int FMT, int D>
__device__ __forceinline__ constexpr int kappa(int kk, int g) {
  if constexpr (FMT == kFmtBf16) {
    return 32 * kk + 8 * g;                        // 16 B of bf16 at 64kk + 16g
  } else if constexpr (FMT == kFmtFp8) {
    return 64 * (kk >> 1) + 16 * g + 8 * (kk & 1); // 16 B of fp8 at 64(kk/2) + 16g
  } else {
    return (D / 4) * g + 8 * kk;                   // 16 B of e2m1 at 16g (D = 128)
  }
}

// Chunks a wave keeps in flight, and waves per SIMD.  bf16 and fp8 pages
// are bound by HBM: two waves holding 32 KB / 24 KB of loads each.  NVFP4
// spends more instructions per byte on dequant, so a third wave (and fewer
// chunks each) hides the dependency stalls better.
template <int FMT>
constexpr int kStages = FMT == kFmtBf16 ? 2 : (FMT == kFmtFp8 ? 3 : 2);
template <int FMT>
constexpr int kWavesPerSimd = FMT == kFmtNvfp4 ? 3 : 2;

template <int FMT, int D>
struct ChunkRaw;

// bf16 pages: each token's D elements (16-token page tiles or K|V rows).
template <int D>
struct ChunkRaw<kFmtBf16, D> {
  static constexpr int KK = D / 32, NN = D / 16;
  u32x4 k[2][KK];          // tile t, step kk: one bf16x8 operand
  uint32_t v[8][NN / 2];   // row i: NN bf16 of columns r*NN ..
};
// fp8 pages: each token's D E4M3FN codes, laid out as for bf16.
template <int D>
struct ChunkRaw<kFmtFp8, D> {
  static constexpr int KK = D / 32, NN = D / 16;
  u32x4 k[2][KK / 2];      // tile t: 16 codes per load = two steps
  uint32_t v[8][NN / 4];   // row i: NN codes
};
// NVFP4 slots (byte order in msa_device.h): K token-major, V in groups of 4 tokens.
template <int D>
struct ChunkRaw<kFmtNvfp4, D> {
  static constexpr int KK = D / 32, NN = D / 16;
  static_assert(D == 128, "NVFP4 attends are built for head_dim 128");
  u32x4 k[2];              // tile t: 32 codes (d in [32g, 32g+32))
  uint32_t ks[2];          // tile t: scales of groups 2g, 2g+1 (low 16 bits)
  uint32_t v[8];           // row i: 8 codes, d in [8r, 8r+8)
  uint32_t vs[2];          // page t: byte i = the scale of group r/2 of token 4g + i
};

// Raw-buffer descriptors (gfx9 layout, unit stride, no swizzle): a load at
// or past num_records bytes returns 0 and touches no memory, which masks the
// tokens past the context and blocks outside the cache without branches.
typedef __amdgpu_buffer_rsrc_t BufRsrc;

__device__ __forceinline__ BufRsrc make_rsrc(const uint8_t* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, bytes, kRawBufferWord3);
}
// AUX is the load's cache policy: 0 normal, kStreamLoads non-temporal
// (lines are not kept for reuse).
constexpr int kStreamLoads = 2;

template <int AUX>
__device__ __forceinline__ u32x4 buf_load16(BufRsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ u32x2 buf_load8(BufRsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ uint32_t buf_load4(BufRsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ uint32_t buf_load2(BufRsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, AUX);
}

// Byte offsets of one lane's loads inside a page tile (bf16 / fp8: the 16
// token rows of one kv head, `rs` bytes apart) or inside an NVFP4 slot's
// code / scale rows.  K: token r of each page; V: tokens 4g .. 4g+3 of each
// page (tau order), columns r*NN .. r*NN + NN.
struct LaneOffsets {
  uint32_t k, v, ks, vs, rs;
};

template <int FMT, int D>
__device__ __forceinline__ LaneOffsets lane_offsets(int lane, int rs) {
  const int r = lane & 15, g = lane >> 4;
  LaneOffsets o;
  if constexpr (FMT == kFmtNvfp4) {
    o.k = r * (D / 2) + 16 * g;           // 32 codes: d in [32g, 32g + 32)
    o.ks = r * (D / 16) + 2 * g;          // scales of groups 2g and 2g + 1
    o.v = (g * (D / 8) + r) * 16;         // 8 codes (d in [8r, 8r + 8)) of tokens 4g .. 4g+3
    o.vs = (g * (D / 16) + (r >> 1)) * 4; // their scales of group r / 2
    o.rs = 0;
  } else {
    constexpr int ESZ = FMT == kFmtBf16 ? 2 : 1, NN = D / 16;
    o.k = r * rs + 16 * g;
    o.v = 4 * g * rs + r * NN * ESZ;
    o.ks = o.vs = 0;
    o.rs = rs;
  }
  return o;
}

// Where chunk c (32 tokens of the row's compacted context: pages 2(c%4) and
// 2(c%4)+1 of block slot c/4) lives.  Wave-uniform.
struct ChunkLoc {
  const uint8_t* k[2];   // K page tiles (NVFP4: K slots) of the two pages
  const uint8_t* v[2];   // V page tiles (NVFP4: V slots)
  int valid[2];          // tokens of each page inside the context; 0 past c_end or outside the cache
  bool ok;               // the block's pages lie inside the cache
};

template <int FMT, int D>
__device__ __forceinline__ ChunkLoc chunk_loc(const AttendArgs& a, const int* slot_list, int c, int c_end, int ctx,
                                              int kvh) {
  ChunkLoc L;
  const bool in = c < c_end;
  const int phys = __builtin_amdgcn_readfirstlane(slot_list[in ? (c >> 2) : 0]);
  const int64_t u0 = (int64_t)phys * a.blk_units + 2 * (c & 3);
  // (the 64-bit compares run on the vector unit: take the verdict back to a scalar)
  L.ok = __builtin_amdgcn_readfirstlane(
      (int)(phys >= 0 && u0 + 1 < a.num_units && (FMT == kFmtNvfp4 || u0 + a.v_unit_offset + 1 < a.num_units)));
  const int rem = ctx - c * 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    L.valid[t] = __builtin_amdgcn_readfirstlane((in && L.ok) ? min(max(rem - 16 * t, 0), kPageTokens) : 0);
    const int64_t off = (u0 + t) * a.sub_stride + (int64_t)kvh * a.head_stride;
    L.k[t] = a.k_base + off;
    L.v[t] = a.v_base + off;
  }
  return L;
}

// Issue every load of one chunk (tokens past the context read as 0).
template <int FMT, int D, int AUX>
__device__ __forceinline__ void issue_loads(ChunkRaw<FMT, D>& raw, const ChunkLoc& L, const LaneOffsets& o) {
  constexpr int KK = D / 32, NN = D / 16;
  if constexpr (FMT == kFmtNvfp4) {
    constexpr int CODE = D / 2, SCALE = D / 16, SREG = kPageTokens * CODE;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const BufRsrc kc = make_rsrc(L.k[t], L.valid[t] * CODE);
      const BufRsrc ksr = make_rsrc(L.k[t] + SREG, L.valid[t] * SCALE);
      raw.k[t] = buf_load16<AUX>(kc, o.k);
      raw.ks[t] = buf_load2<AUX>(ksr, o.ks);
    }
    // V slots interleave the tokens of a group of 4, so a descriptor covers
    // a whole page whenever any of it is valid; the scales of tokens past the
    // context are cleared in the context's last chunk instead (codes are
    // always finite, an unwritten scale byte may not be)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool any = L.valid[t] > 0;
      const BufRsrc vc = make_rsrc(L.v[t], any ? kPageTokens * CODE : 0);
      const BufRsrc vsr = make_rsrc(L.v[t] + SREG, any ? kPageTokens * SCALE : 0);
      const u32x4 w = buf_load16<AUX>(vc, o.v);
      raw.v[4 * t + 0] = w[0];
      raw.v[4 * t + 1] = w[1];
      raw.v[4 * t + 2] = w[2];
      raw.v[4 * t + 3] = w[3];
      raw.vs[t] = buf_load4<AUX>(vsr, o.vs);
    }
  } else {
    // A descriptor ends with the last valid token's row piece: rows past it
    // (and, in K|V-interleaved rows, the other side's half) read as 0.
    constexpr int ESZ = FMT == kFmtBf16 ? 2 : 1, ROW = D * ESZ;
    const int rs = o.rs;
    int span[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) span[t] = L.valid[t] > 0 ? (L.valid[t] - 1) * rs + ROW : 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const BufRsrc kr = make_rsrc(L.k[t], span[t]);
      if constexpr (FMT == kFmtBf16) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) raw.k[t][kk] = buf_load16<AUX>(kr, o.k + 64 * kk);
      } else {
#pragma unroll
        for (int kp = 0; kp < KK / 2; ++kp) raw.k[t][kp] = buf_load16<AUX>(kr, o.k + 64 * kp);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const BufRsrc vr = make_rsrc(L.v[t], span[t]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t* dst = raw.v[4 * t + i];
        constexpr int W = NN * ESZ / 4;   // dwords of one lane's row piece
        if constexpr (W == 4) {
          const u32x4 x = buf_load16<AUX>(vr, o.v + i * rs);
          dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
        } else if constexpr (W == 2) {
          const u32x2 x = buf_load8<AUX>(vr, o.v + i * rs);
          dst[0] = x[0]; dst[1] = x[1];
        } else {
          dst[0] = buf_load4<AUX>(vr, o.v + i * rs);
        }
      }
    }
  }
}

// Operand types.  QK^T: bf16 for bf16 / fp8 pages, fp16 for NVFP4 pages (the
// query is converted once).  PV: fp16 wherever V is exact in fp16 (E4M3 and
// e2m1 x E4M3 values are), so the probabilities keep 11 significant bits
// instead of bf16's 8; bf16 pages keep bf16 V and probabilities (bf16's
// range is wider than fp16's).
template <int FMT> struct OpType { typedef bf16x8 type; };
template <> struct OpType<kFmtNvfp4> { typedef f16x8 type; };
template <int FMT> struct PvType { typedef f16x8 type; };
template <> struct PvType<kFmtBf16> { typedef bf16x8 type; };

// K operand of tile t, step kk.
template <int FMT, int D>
__device__ __forceinline__ typename OpType<FMT>::type k_operand(const ChunkRaw<FMT, D>& raw, int t, int kk) {
  typedef typename OpType<FMT>::type OT;
  if constexpr (FMT == kFmtBf16) {
    return __builtin_bit_cast(OT, raw.k[t][kk]);
  } else if constexpr (FMT == kFmtFp8) {
    const u32x4 w = raw.k[t][kk >> 1];
    const uint32_t w0 = (kk & 1) ? w[2] : w[0], w1 = (kk & 1) ? w[3] : w[1];
    u32x4 o = {fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
               fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)};
    return __builtin_bit_cast(OT, o);
  } else {
    const uint32_t w = raw.k[t][kk];
    const f16x2 sc = fp8x2_to_f16x2<false>(raw.ks[t]);          // (scale 2g, scale 2g+1)
    const f16x2 s = kk < 2 ? f16x2{sc[0], sc[0]} : f16x2{sc[1], sc[1]};
    u32x4 o = {f16x2_bits(fp4x2_to_f16x2<0>(w) * s), f16x2_bits(fp4x2_to_f16x2<1>(w) * s),
               f16x2_bits(fp4x2_to_f16x2<2>(w) * s), f16x2_bits(fp4x2_to_f16x2<3>(w) * s)};
    return __builtin_bit_cast(OT, o);
  }
}

// V^T operands: vop[nn] holds, for lane (r, g), column d = r*NN + nn of the
// token rows tau(8g + 0 .. 7), as pairs (row 2p, row 2p+1).  The pairs are
// formed on the raw codes where that is cheaper than on converted values:
// a byte permute for fp8, a nibble merge for NVFP4 (one e2m1 byte then
// converts straight into a (row 2p, row 2p+1) pair).
template <int FMT, int D>
__device__ __forceinline__ void v_operands(const ChunkRaw<FMT, D>& raw, u32x4 vop[D / 16]) {
  constexpr int NN = D / 16;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if constexpr (FMT == kFmtBf16) {
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        const uint32_t a0 = raw.v[2 * p][nn >> 1], a1 = raw.v[2 * p + 1][nn >> 1];
        vop[nn][p] = (nn & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
      }
    } else if constexpr (FMT == kFmtFp8) {
#pragma unroll
      for (int w = 0; w < NN / 4; ++w) {
        const uint32_t a = raw.v[2 * p][w], b = raw.v[2 * p + 1][w];
        // (a0, b0, a1, b1) and (a2, b2, a3, b3)
        const uint32_t lo = (a & 0xffu) | ((b & 0xffu) << 8) | ((a & 0xff00u) << 8) | ((b & 0xff00u) << 16);
        const uint32_t hi = ((a >> 16) & 0xffu) | ((b >> 8) & 0xff00u) | ((a >> 8) & 0xff0000u) | (b & 0xff000000u);
        vop[4 * w + 0][p] = f16x2_bits(fp8x2_to_f16x2<false>(lo));
        vop[4 * w + 1][p] = f16x2_bits(fp8x2_to_f16x2<true>(lo));
        vop[4 * w + 2][p] = f16x2_bits(fp8x2_to_f16x2<false>(hi));
        vop[4 * w + 3][p] = f16x2_bits(fp8x2_to_f16x2<true>(hi));
      }
    } else {
      const uint32_t a = raw.v[2 * p], b = raw.v[2 * p + 1];
      // (scale a, scale b): bytes 2 (p % 2), 2 (p % 2) + 1 of page p / 2's scale word
      const f16x2 s = (p & 1) ? fp8x2_to_f16x2<true>(raw.vs[p >> 1]) : fp8x2_to_f16x2<false>(raw.vs[p >> 1]);
      // byte j of x: element 2j of a (low nibble) and of b (high nibble); y: element 2j + 1
      const uint32_t x = (a & 0x0f0f0f0fu) | ((b << 4) & 0xf0f0f0f0u);
      const uint32_t y = ((a >> 4) & 0x0f0f0f0fu) | (b & 0xf0f0f0f0u);
      vop[0][p] = f16x2_bits(fp4x2_to_f16x2<0>(x) * s);
      vop[2][p] = f16x2_bits(fp4x2_to_f16x2<1>(x) * s);
      vop[4][p] = f16x2_bits(fp4x2_to_f16x2<2>(x) * s);
      vop[6][p] = f16x2_bits(fp4x2_to_f16x2<3>(x) * s);
      vop[1][p] = f16x2_bits(fp4x2_to_f16x2<0>(y) * s);
      vop[3][p] = f16x2_bits(fp4x2_to_f16x2<1>(y) * s);
      vop[5][p] = f16x2_bits(fp4x2_to_f16x2<2>(y) * s);
      vop[7][p] = f16x2_bits(fp4x2_to_f16x2<3>(y) * s);
    }
  }
}

// NVFP4 V slots are read whole (their tokens are interleaved by 4), so in a
// context's last chunk the scales of tokens at or past lim are cleared before
// conversion: their codes are finite, an unwritten scale byte may not be.
// Lane (r, g) holds the scale bytes of tokens tok0 + 16 t + i (i < 4) of page t.
template <int D>
__device__ __forceinline__ void nvfp4_clear_v_scales(ChunkRaw<kFmtNvfp4, D>& rv, int tok0, int lim) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t keep = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) keep |= (tok0 + 16 * t + i < lim) ? (0xffu << (8 * i)) : 0u;
    rv.vs[t] &= keep;
  }
}

template <int FMT, int D>
struct WaveState {
  static constexpr int NN = D / 16;
  f32x4 acc[NN];
  f32x4 lacc;  // softmax denominator: P times an all-ones operand (every entry = the head's sum)
  float m;     // reference max (log2 units), the same on the 4 lanes of a head
};

// The online softmax rescales only when some lane's chunk max exceeds the
// reference by more than kLazy (log2 units): probabilities stay below 2^kLazy
// and the common case needs neither a cross-lane max nor a rescale.
constexpr float kLazyMax = 8.f;

// One 32-token chunk of one wave, from registers already loaded.  Scores of
// tokens at or past `lim` are masked when `masked` (the context's last chunk,
// or a block outside the cache, for which lim is 0).
template <int FMT, int D>
__device__ __forceinline__ void compute_chunk(WaveState<FMT, D>& st, const ChunkRaw<FMT, D>& raw,
                                              const typename OpType<FMT>::type* qop, float sl2, bool masked,
                                              int tok0, int lim) {
  constexpr int KK = D / 32, NN = D / 16;
  typedef typename OpType<FMT>::type OT;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    s0 = mfma16(k_operand<FMT, D>(raw, 0, kk), qop[kk], s0);
    s1 = mfma16(k_operand<FMT, D>(raw, 1, kk), qop[kk], s1);
  }
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = s0[i];
    sc[4 + i] = s1[i];
  }
  if (masked) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = tok0 + i < lim ? sc[i] : -INFINITY;
      sc[4 + i] = tok0 + 16 + i < lim ? sc[4 + i] : -INFINITY;
    }
  }
  float mx = sc[0];   // IEEE maximum: v_maximum3, no NaN-quieting moves
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = __builtin_elementwise_maximum(mx, sc[i]);
  const float mxs = mx * sl2;
  if (__ballot(mxs > st.m + kLazyMax)) {   // rare after the first chunk
    float mh = fmaxf(mxs, __shfl_xor(mxs, 16));
    mh = fmaxf(mh, __shfl_xor(mh, 32));
    const float m_new = fmaxf(st.m, mh);
    const float alpha = exp2_fast(st.m - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) st.acc[nn] = st.acc[nn] * alpha;
    st.lacc = st.lacc * alpha;
    st.m = m_new;
  }
  const float off = -(st.m == -INFINITY ? 0.f : st.m);
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = exp2_fast(fmaf(sc[i], sl2, off));
  typedef typename PvType<FMT>::type PT;
  u32x4 pw, onesw;
  if constexpr (FMT != kFmtBf16) {
    pw = u32x4{pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]), pack_f16(p[6], p[7])};
    onesw = u32x4{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
  } else {
    pw = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
    onesw = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  }
  const PT pop = __builtin_bit_cast(PT, pw);
  u32x4 vop[NN];
  if constexpr (FMT == kFmtNvfp4) {
    ChunkRaw<FMT, D> rv = raw;
    if (masked) nvfp4_clear_v_scales(rv, tok0, lim);
    v_operands<FMT, D>(rv, vop);
  } else {
    v_operands<FMT, D>(raw, vop);
  }
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) st.acc[nn] = mfma16(__builtin_bit_cast(PT, vop[nn]), pop, st.acc[nn]);
  st.lacc = mfma16(__builtin_bit_cast(PT, onesw), pop, st.lacc);
}

// Shared memory of one workgroup.
// One unit's LDS: its slot list and the merge area of its (up to) NW waves.
template <int D, int NW>
struct AttendSmem {
  int slot_list[kMaxTopK];
  int ctx;
  float m[NW][16];
  float l[NW][16];
  float o[NW][16][D];
};

// UPW units (row, kv head, split) per workgroup.  UPW = 1: the workgroup's
// 3 or 4 waves (blockDim) all serve its unit.  UPW = 4 (NVFP4 pages): 3 waves
// per unit, 12 per workgroup, so that a workgroup fills one CU at 3 waves per
// SIMD and the LDS of four units keeps a second one off it: the grid is
// placed whole in one round.  (Separate 3-wave workgroups leave some SIMDs
// with fewer waves than others, and on a machine filled to 3 per SIMD a few
// workgroups then find no SIMDs to start on until others finish.)  Units past
// the last one take part in the barriers only.
template <int FMT, int D, int AUX, int UPW>
__global__ __launch_bounds__(UPW == 1 ? 256 : 192 * UPW, kWavesPerSimd<FMT>) void attend_rows_kernel(const AttendArgs a) {
  constexpr int KK = D / 32, NN = D / 16, NB = kStages<FMT>;
  constexpr int NWMAX = UPW == 1 ? 4 : 3;
  typedef typename OpType<FMT>::type OT;
  __shared__ AttendSmem<D, NWMAX> smem[UPW];
  const int wave_wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // waves per unit (3 or 4), this wave's unit and its index among the unit's waves
  const int nw = UPW == 1 ? __builtin_amdgcn_readfirstlane(blockDim.x >> 6) : 3;
  const int unit = UPW == 1 ? 0 : wave_wg / 3;
  const int wave = wave_wg - unit * nw;
  AttendSmem<D, NWMAX>& sm = smem[unit];
  const int r = lane & 15, g = lane >> 4;
  const int64_t units = (int64_t)a.total_rows * a.num_kv_heads * a.nsplit;
  const int64_t uid = (int64_t)blockIdx.x * UPW + unit;
  const bool live = uid < units;
  int bid = (int)(live ? uid : 0);
  const int split = bid % a.nsplit;
  bid /= a.nsplit;
  const int kvh = bid % a.num_kv_heads;
  const int row = bid / a.num_kv_heads;

  int req, abs_pos;
  decode_row_position(a.seq_lens, a.dql, row, &req, &abs_pos);
  // Q operand rows (head kvh*G + r; padded heads r >= G read head kvh*G
  // and drop it, so no load is lane-masked).  bf16 and fp8 pages load them,
  // and k_scale, before the row's compaction, which their latency then
  // overlaps, so that the waits for them cover no chunk load (measured up
  // to 3 % faster at C3, level at C2).  NVFP4 loads them after its first
  // chunks: loading them early measured 2 % slower at C5.
  const int G = a.group;
  constexpr bool kEarlyQ = FMT != kFmtNvfp4;
  const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                        ((int64_t)row * a.num_q_heads + kvh * G + (r < G ? r : 0)) * D * 2;
  u32x4 qraw[KK];
  float kscale = 1.f;
  if constexpr (kEarlyQ) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qraw[kk] = *reinterpret_cast<const u32x4*>(qrow + 2 * kappa<FMT, D>(kk, g));
    kscale = a.k_scale ? *a.k_scale : 1.f;
  }
  if (wave == 0) {
    const RowSlots rs = compact_row(a.topk + (int64_t)row * a.topk_stride, a.topk_k,
                                    a.block_table + (int64_t)req * a.bt_stride, a.bt_cols, abs_pos, sm.slot_list);
    if (lane == 0) sm.ctx = rs.ctx;
  }
  __syncthreads();
  const int ctx = live ? __builtin_amdgcn_readfirstlane(sm.ctx) : 0;
  const int nchunks = (ctx + 31) >> 5;
  const int c0 = (int)((int64_t)nchunks * split / a.nsplit);
  const int c1 = (int)((int64_t)nchunks * (split + 1) / a.nsplit);

  // this wave's chunks: cw, cw + nw, cw + 2 nw, ... below c1; NB of them in flight
  const LaneOffsets lo = lane_offsets<FMT, D>(lane, a.row_stride);
  const int cw = c0 + wave;
  const int n_w = cw < c1 ? (c1 - cw + nw - 1) / nw : 0;
  ChunkRaw<FMT, D> raw[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    issue_loads<FMT, D, AUX>(raw[b], chunk_loc<FMT, D>(a, sm.slot_list, cw + nw * b, c1, ctx, kvh), lo);
  asm volatile("" ::: "memory");


  if constexpr (!kEarlyQ) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qraw[kk] = *reinterpret_cast<const u32x4*>(qrow + 2 * kappa<FMT, D>(kk, g));
    kscale = a.k_scale ? *a.k_scale : 1.f;
  }
  OT qop[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 w = r < G ? qraw[kk] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (FMT == kFmtNvfp4) {
      w = u32x4{bf16x2_to_f16x2(w[0]), bf16x2_to_f16x2(w[1]), bf16x2_to_f16x2(w[2]), bf16x2_to_f16x2(w[3])};
    }
    qop[kk] = __builtin_bit_cast(OT, w);
  }
  const float sl2 = a.softmax_scale * kscale * kLog2e;

  WaveState<FMT, D> st;
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) st.acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.lacc = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;

  // Loads are issued unconditionally (past the wave's range they fetch
  // nothing), so every path has the same outstanding loads and each chunk
  // waits only for its own.
  for (int j = 0; j < n_w; j += NB) {
    if constexpr (UPW > 1) {
      // One-round grid: all waves start together and the launch ends with
      // the last.  Issue priority by remaining work (3 for the first quarter
      // of a wave's chunks, down to 0 for the last) lets lagging waves issue
      // before leading ones; by default the oldest waves of a CU win issue
      // and finish far ahead of the youngest.
      const int p = min(3, (4 * (n_w - j)) / n_w);
      if (p == 3) __builtin_amdgcn_s_setprio(3);
      else if (p == 2) __builtin_amdgcn_s_setprio(2);
      else if (p == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = cw + nw * (j + b);
      if (j + b < n_w) {
        const ChunkLoc L = chunk_loc<FMT, D>(a, sm.slot_list, c, c1, ctx, kvh);
        const bool masked = !L.ok || c * 32 + 32 > ctx;
        compute_chunk<FMT, D>(st, raw[b], qop, sl2, masked, c * 32 + 4 * g, L.ok ? ctx : 0);
      }
      issue_loads<FMT, D, AUX>(raw[b], chunk_loc<FMT, D>(a, sm.slot_list, c + nw * NB, c1, ctx, kvh), lo);
      // keep these loads here, NB chunks ahead of their use: the compiler
      // may not sink them towards the chunk that reads them
      asm volatile("" ::: "memory");
    }
  }

  if constexpr (UPW > 1) __builtin_amdgcn_s_setprio(0);
  // merge the waves through LDS
  const float lsum = st.lacc[0];
  if (r < G) {
    if (g == 0) {
      sm.m[wave][r] = st.m;
      sm.l[wave][r] = lsum;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) sm.o[wave][r][(4 * g + i) * NN + nn] = st.acc[nn][i];
    }
  }
  __syncthreads();
  const float vscale = a.v_scale ? *a.v_scale : 1.f;
  for (int idx = wave * 64 + lane; live && idx < G * (D / 4); idx += nw * 64) {
    const int h = idx / (D / 4), d = (idx % (D / 4)) * 4;
    float M = sm.m[0][h];
#pragma unroll
    for (int w = 1; w < NWMAX; ++w)
      if (w < nw) M = fmaxf(M, sm.m[w][h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) {
      if (w >= nw) break;
      const float e = exp2_fast(sm.m[w][h] - Mu);
      L += sm.l[w][h] * e;
      o0 += sm.o[w][h][d] * e;
      o1 += sm.o[w][h][d + 1] * e;
      o2 += sm.o[w][h][d + 2] * e;
      o3 += sm.o[w][h][d + 3] * e;
    }
    const int qh = kvh * G + h;
    if (a.nsplit == 1) {
      const float inv = L > 0.f ? vscale / L : 0.f;
      uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.out) +
                                                  (((int64_t)row * a.num_q_heads + qh) * D + d) * 2);
      dst[0] = pack_bf16(o0 * inv, o1 * inv);
      dst[1] = pack_bf16(o2 * inv, o3 * inv);
    } else {
      const int64_t part = ((int64_t)row * a.num_q_heads + qh) * a.nsplit + split;
      f32x4* po = reinterpret_cast<f32x4*>(a.ws_o + part * D + d);
      *po = f32x4{o0, o1, o2, o3};
      if (d == 0) {
        a.ws_ml[2 * part] = M;
        a.ws_ml[2 * part + 1] = L;
      }
    }
  }
}

// Combine split partials: one thread per 4 output elements of a (row, head).
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(const AttendArgs a, int pairs) {
  const int per_pair = D / 4;
  const int pair = blockIdx.x * (256 / per_pair) + threadIdx.x / per_pair;
  if (pair >= pairs) return;
  const int d = (threadIdx.x % per_pair) * 4;
  const int ns = a.nsplit;
  const int64_t base = (int64_t)pair * ns;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_ml[2 * (base + s)]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const float e = exp2_fast(a.ws_ml[2 * (base + s)] - Mu);
    L += a.ws_ml[2 * (base + s) + 1] * e;
    o += *reinterpret_cast<const f32x4*>(a.ws_o + (base + s) * D + d) * e;
  }
  const float vscale = a.v_scale ? *a.v_scale : 1.f;
  const float inv = L > 0.f ? vscale / L : 0.f;
  uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.out) + ((int64_t)pair * D + d) * 2);
  dst[0] = pack_bf16(o[0] * inv, o[1] * inv);
  dst[1] = pack_bf16(o[2] * inv, o[3] * inv);
}

// ---------------------------------------------------------------------------
// Test hook: each row's K and V in sparse-table order, exactly as the decode
// attend's gather produces its matrix operands.  One wave per (row, kv head)
// walks the row's 32-token chunks with the attend's own chunk_loc /
// issue_loads, converts with k_operand / v_operands (and, for NVFP4, the same
// V-scale clearing in the context's last chunk), and writes each operand
// element, times k_scale or v_scale in fp32, at its token and d.  Token t of
// the row is slot t / 128 of sparse_bt (its physical block is the slot's first
// page id / block_page_stride); tokens at or past ctx are 0.
// out[row][token][kv head][d], width_tokens tokens per row.
// ---------------------------------------------------------------------------
template <int FMT, int D>
__global__ __launch_bounds__(64) void gather_dequant_decode_kernel(const AttendArgs a, const int32_t* __restrict__ sbt,
                                                                   int64_t sbt_stride, const int32_t* __restrict__ sctx,
                                                                   int bps, int width_tokens, float* __restrict__ k_out,
                                                                   float* __restrict__ v_out) {
  constexpr int KK = D / 32, NN = D / 16;
  typedef typename OpType<FMT>::type OT;
  typedef typename PvType<FMT>::type PT;
  __shared__ int slot_list[kMaxTopK];
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int64_t row = blockIdx.x / a.num_kv_heads;
  const int ctx = min(max(sctx[row], 0), width_tokens);
  const int nslots = (ctx + kBlockTokens - 1) / kBlockTokens;
  for (int s = lane; s < nslots; s += 64) slot_list[s] = sbt[row * sbt_stride + kPagesPerBlock * s] / bps;
  __syncthreads();
  const int nchunks = (ctx + 31) >> 5;
  const LaneOffsets lo = lane_offsets<FMT, D>(lane, a.row_stride);
  const float ks = a.k_scale ? *a.k_scale : 1.f, vs = a.v_scale ? *a.v_scale : 1.f;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;
  float* kb = k_out + (row * width_tokens * a.num_kv_heads + kvh) * D;
  float* vb = v_out + (row * width_tokens * a.num_kv_heads + kvh) * D;
  for (int c = 0; c < nchunks; ++c) {
    ChunkRaw<FMT, D> raw;
    const ChunkLoc L = chunk_loc<FMT, D>(a, slot_list, c, nchunks, ctx, kvh);
    issue_loads<FMT, D, 0>(raw, L, lo);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const OT op = k_operand<FMT, D>(raw, t, kk);
        float* dst = kb + (int64_t)(c * 32 + 16 * t + r) * tok_stride + kappa<FMT, D>(kk, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = (float)op[e] * ks;
      }
    }
    const bool masked = !L.ok || c * 32 + 32 > ctx;
    u32x4 vop[NN];
    if constexpr (FMT == kFmtNvfp4) {
      ChunkRaw<FMT, D> rv = raw;
      if (masked) nvfp4_clear_v_scales(rv, c * 32 + 4 * g, L.ok ? ctx : 0);
      v_operands<FMT, D>(rv, vop);
    } else {
      v_operands<FMT, D>(raw, vop);
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const PT op = __builtin_bit_cast(PT, vop[nn]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // row i of the operand: chunk token tau(8g + i)
        const int tok = c * 32 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
        vb[(int64_t)tok * tok_stride + r * NN + nn] = (float)op[i] * vs;
      }
    }
  }
  // slots past the context
  for (int idx = nchunks * 32 * D + lane; idx < width_tokens * D; idx += 64) {
    const int64_t off = (int64_t)(idx / D) * tok_stride + idx % D;
    kb[off] = 0.f;
    vb[off] = 0.f;
  }
}

hipError_t launch_gather_dequant_decode(const AttendArgs& a, int fmt, const int32_t* sbt, int64_t sbt_stride,
                                        const int32_t* sctx, int bps, int rows, int width_tokens, float* k_out,
                                        float* v_out, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)rows * a.num_kv_heads)), block(64);
  log_launch("gather_dequant_decode_kernel head_dim %d: %d rows x %d kv heads, %d tokens per row", a.head_dim, rows,
             a.num_kv_heads, width_tokens);
  if (a.head_dim == 128) {
    if (fmt == kFmtBf16)
      hipLaunchKernelGGL((gather_dequant_decode_kernel<kFmtBf16, 128>), grid, block, 0, stream, a, sbt, sbt_stride,
                         sctx, bps, width_tokens, k_out, v_out);
    else if (fmt == kFmtFp8)
      hipLaunchKernelGGL((gather_dequant_decode_kernel<kFmtFp8, 128>), grid, block, 0, stream, a, sbt, sbt_stride,
                         sctx, bps, width_tokens, k_out, v_out);
    else
      hipLaunchKernelGGL((gather_dequant_decode_kernel<kFmtNvfp4, 128>), grid, block, 0, stream, a, sbt, sbt_stride,
                         sctx, bps, width_tokens, k_out, v_out);
  } else {
    if (fmt == kFmtBf16)
      hipLaunchKernelGGL((gather_dequant_decode_kernel<kFmtBf16, 64>), grid, block, 0, stream, a, sbt, sbt_stride,
                         sctx, bps, width_tokens, k_out, v_out);
    else
      hipLaunchKernelGGL((gather_dequant_decode_kernel<kFmtFp8, 64>), grid, block, 0, stream, a, sbt, sbt_stride,
                         sctx, bps, width_tokens, k_out, v_out);
  }
  return hipGetLastError();
}

// Waves per workgroup: 4 unless fewer waves fill the machine in fewer,
// fuller rounds.  A CU holds waves_per_simd * 4 waves and at most 4
// workgroups (LDS); a workgroup of nw waves takes nw of those slots.
static int choose_waves(int64_t units, int waves_per_simd, int cus) {
  int best = 4;
  double best_util = 0.0;
  for (int nw = 4; nw >= 3; --nw) {
    const int64_t per_cu = std::min<int64_t>(4, (4 * waves_per_simd) / nw);
    const int64_t per_round = per_cu * (cus > 0 ? cus : 256);
    const int64_t rounds = (units + per_round - 1) / per_round;
    const double util = (double)units / (double)(rounds * per_round);
    if (util > best_util + 1e-9) {
      best_util = util;
      best = nw;
    }
  }
  return best;
}

// Units per workgroup: 4 (3 waves each) for a grid of 3-wave units that
// needs more than 3 and at most 4 per CU, which then runs as one 12-wave
// workgroup per CU; 1 otherwise.
static int choose_units_per_wg(int64_t units, int nw, int cus) {
  const int64_t c = cus > 0 ? cus : 256;
  return nw == 3 && units > 3 * c && units <= 4 * c ? 4 : 1;
}

template <int FMT, int D>
static hipError_t launch_fmt(const AttendArgs& a, int rows, hipStream_t stream) {
  const int64_t units = (int64_t)rows * a.num_kv_heads * a.nsplit;
  const int nw = choose_waves(units, kWavesPerSimd<FMT>, a.num_cus);
  const int upw = kWavesPerSimd<FMT> >= 3 ? choose_units_per_wg(units, nw, a.num_cus) : 1;
  const unsigned grid = (unsigned)((units + upw - 1) / upw);
  // With one query row per request each page is read by exactly one
  // workgroup: stream it past the caches.  Several rows of a request (a
  // multi-token decode) select overlapping blocks, which the L2 then serves
  // to the neighbouring rows.
  const bool streamed = a.dql == 1;
  log_launch("attend_rows_kernel decode, %s pages, head_dim %d: %lld units (row x kv head x split) of %d waves, "
             "%d per workgroup (%u workgroups), %d split%s, %s loads",
             FMT == kFmtBf16 ? "bf16" : (FMT == kFmtFp8 ? "fp8" : "nvfp4"), D, (long long)units, nw, upw, grid,
             a.nsplit, a.nsplit == 1 ? "" : "s", streamed ? "streaming" : "cached");
  if (upw == 4) {
    if constexpr (kWavesPerSimd<FMT> >= 3) {
      if (streamed)
        hipLaunchKernelGGL((attend_rows_kernel<FMT, D, kStreamLoads, 4>), dim3(grid), dim3(64 * 3 * 4), 0, stream, a);
      else
        hipLaunchKernelGGL((attend_rows_kernel<FMT, D, 0, 4>), dim3(grid), dim3(64 * 3 * 4), 0, stream, a);
    }
  } else if (streamed) {
    hipLaunchKernelGGL((attend_rows_kernel<FMT, D, kStreamLoads, 1>), dim3(grid), dim3(64 * nw), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attend_rows_kernel<FMT, D, 0, 1>), dim3(grid), dim3(64 * nw), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int pairs = rows * a.num_q_heads;
  const int per_block = 256 / (D / 4);
  log_launch("attend_merge_kernel head_dim %d: %d (row, head) pairs, %d splits", D, pairs, a.nsplit);
  hipLaunchKernelGGL((attend_merge_kernel<D>), dim3((unsigned)((pairs + per_block - 1) / per_block)), dim3(256), 0,
                     stream, a, pairs);
  return hipGetLastError();
}

hipError_t launch_attend_decode(const AttendArgs& a, int fmt, int rows, hipStream_t stream) {
  if (a.head_dim == 128) {
    if (fmt == kFmtBf16) return launch_fmt<kFmtBf16, 128>(a, rows, stream);
    if (fmt == kFmtFp8) return launch_fmt<kFmtFp8, 128>(a, rows, stream);
    return launch_fmt<kFmtNvfp4, 128>(a, rows, stream);
  }
  if (fmt == kFmtBf16) return launch_fmt<kFmtBf16, 64>(a, rows, stream);
  return launch_fmt<kFmtFp8, 64>(a, rows, stream);
}

}  // namespace msa
