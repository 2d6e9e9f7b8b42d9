// Row-wise block-sparse attend over a paged KV cache (decode, and prefill
// rows taken one at a time).
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
// Work decomposition.  One workgroup (4 waves) owns (row, kv head, split).
// Wave 0 compacts the row's top-k ids into the slot list (full blocks, then
// the causal tail) in LDS.  The row's context [0, ctx) is cut into 32-token
// chunks (two 16-token pages of one 128-token block); a split owns a
// contiguous range of chunks and its four waves take every fourth chunk.
// Each wave keeps its own online-softmax state, loads the next chunk while it
// computes the current one, and the four states are merged through LDS at
// the end.  With one split the workgroup writes the bf16 output directly;
// otherwise it writes an fp32 partial (o, m, l) and attend_merge combines.
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

template <int FMT, int D>
struct ChunkRaw;

// bf16 pages: [page][Hkv][16][D] bf16.
template <int D>
struct ChunkRaw<kFmtBf16, D> {
  static constexpr int KK = D / 32, NN = D / 16;
  u32x4 k[2][KK];          // tile t, step kk: one bf16x8 operand
  uint32_t v[8][NN / 2];   // row i: NN bf16 of columns r*NN ..
};
// fp8 pages: [page][Hkv][16][D] E4M3FN codes.
template <int D>
struct ChunkRaw<kFmtFp8, D> {
  static constexpr int KK = D / 32, NN = D / 16;
  u32x4 k[2][KK / 2];      // tile t: 16 codes per load = two steps
  uint32_t v[8][NN / 4];   // row i: NN codes
};
// NVFP4 slots: per token D/2 code bytes, then per token D/16 scale bytes.
template <int D>
struct ChunkRaw<kFmtNvfp4, D> {
  static constexpr int KK = D / 32, NN = D / 16;
  static_assert(D == 128, "NVFP4 attends are built for head_dim 128");
  u32x4 k[2];              // tile t: 32 codes (d in [32g, 32g+32))
  uint32_t ks[2];          // tile t: scales of groups 2g, 2g+1 (low 16 bits)
  uint32_t v[8];           // row i: 8 codes, d in [8r, 8r+8)
  uint32_t vs[8];          // row i: the scale of group r/2 (low 8 bits)
};

template <class T>
__device__ __forceinline__ T load_or_zero(bool ok, const void* p) {
  T z;
  __builtin_memset(&z, 0, sizeof(T));
  return ok ? *reinterpret_cast<const T*>(p) : z;
}

// Where chunk c (32 tokens of the row's compacted context) lives.
struct ChunkAddr {
  int64_t pg0;      // K page of the chunk's first 16 tokens (the next page holds the rest)
  int64_t vpg0;     // V page (bf16 / fp8: pg0 + the V page offset)
  bool ok;          // the block's pages lie inside the cache
};

template <int FMT>
__device__ __forceinline__ ChunkAddr chunk_addr(const AttendArgs& a, const int* slot_list, int c) {
  const int phys = __builtin_amdgcn_readfirstlane(slot_list[c >> 2]);
  ChunkAddr ca;
  ca.pg0 = (int64_t)phys * a.block_page_stride + 2 * (c & 3);
  ca.vpg0 = ca.pg0 + a.v_page_offset;
  ca.ok = phys >= 0 && ca.pg0 + 1 < a.num_pages && (FMT == kFmtNvfp4 || ca.vpg0 + 1 < a.num_pages);
  return ca;
}

// K half of chunk c (tokens past ctx, or of a block outside the cache, read as 0).
template <int FMT, int D>
__device__ __forceinline__ void load_k(ChunkRaw<FMT, D>& raw, const AttendArgs& a, const ChunkAddr& ca, int c,
                                       int ctx, int kvh, int lane) {
  constexpr int KK = D / 32;
  const int r = lane & 15, g = lane >> 4;
  const int tok0 = c * 32;
  if constexpr (FMT == kFmtNvfp4) {
    constexpr int SLOT = 9 * D, CODE_ROW = D / 2, SCALE_ROW = D / 16;
    const uint8_t* kslot = a.k_base + ca.pg0 * a.page_stride + (int64_t)(2 * kvh) * SLOT;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool ok = ca.ok && tok0 + 16 * t + r < ctx;
      const uint8_t* s = kslot + t * a.page_stride;
      raw.k[t] = load_or_zero<u32x4>(ok, s + r * CODE_ROW + 16 * g);
      raw.ks[t] = ok ? (uint32_t) * reinterpret_cast<const uint16_t*>(s + 16 * CODE_ROW + r * SCALE_ROW + 2 * g) : 0u;
    }
  } else {
    constexpr int ROW = D * (FMT == kFmtBf16 ? 2 : 1);
    const uint8_t* kp = a.k_base + ca.pg0 * a.page_stride + (int64_t)kvh * kPageTokens * ROW;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool ok = ca.ok && tok0 + 16 * t + r < ctx;
      const uint8_t* row = kp + t * a.page_stride + r * ROW;
      if constexpr (FMT == kFmtBf16) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) raw.k[t][kk] = load_or_zero<u32x4>(ok, row + 2 * kappa<FMT, D>(kk, g));
      } else {
#pragma unroll
        for (int kp2 = 0; kp2 < KK / 2; ++kp2) raw.k[t][kp2] = load_or_zero<u32x4>(ok, row + kappa<FMT, D>(2 * kp2, g));
      }
    }
  }
}

// V half of chunk c: lane (r, g) takes token rows tau(8g + i) (4g + i of the
// first page for i < 4, 4g + i - 4 of the second), columns r * NN .. + NN.
template <int FMT, int D>
__device__ __forceinline__ void load_v(ChunkRaw<FMT, D>& raw, const AttendArgs& a, const ChunkAddr& ca, int c,
                                       int ctx, int kvh, int lane) {
  constexpr int NN = D / 16;
  const int r = lane & 15, g = lane >> 4;
  const int tok0 = c * 32;
  if constexpr (FMT == kFmtNvfp4) {
    constexpr int SLOT = 9 * D, CODE_ROW = D / 2, SCALE_ROW = D / 16;
    const uint8_t* vslot = a.k_base + ca.pg0 * a.page_stride + (int64_t)(2 * kvh + 1) * SLOT;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
      const bool ok = ca.ok && tok0 + t < ctx;
      const uint8_t* s = vslot + (t >> 4) * a.page_stride;
      const int tr = t & 15;
      raw.v[i] = load_or_zero<uint32_t>(ok, s + tr * CODE_ROW + 4 * r);
      raw.vs[i] = ok ? (uint32_t)s[16 * CODE_ROW + tr * SCALE_ROW + (r >> 1)] : 0u;
    }
  } else {
    constexpr int ESZ = FMT == kFmtBf16 ? 2 : 1;
    constexpr int ROW = D * ESZ;
    const uint8_t* vp = a.v_base + ca.vpg0 * a.page_stride + (int64_t)kvh * kPageTokens * ROW;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
      const bool ok = ca.ok && tok0 + t < ctx;
      const uint8_t* row = vp + (t >> 4) * a.page_stride + (t & 15) * ROW + r * NN * ESZ;
      if constexpr (FMT == kFmtBf16) {
        if constexpr (NN / 2 == 4) {
          const u32x4 x = load_or_zero<u32x4>(ok, row);
          raw.v[i][0] = x[0]; raw.v[i][1] = x[1]; raw.v[i][2] = x[2]; raw.v[i][3] = x[3];
        } else {
          const u32x2 x = load_or_zero<u32x2>(ok, row);
          raw.v[i][0] = x[0]; raw.v[i][1] = x[1];
        }
      } else {
        if constexpr (NN / 4 == 2) {
          const u32x2 x = load_or_zero<u32x2>(ok, row);
          raw.v[i][0] = x[0]; raw.v[i][1] = x[1];
        } else {
          raw.v[i][0] = load_or_zero<uint32_t>(ok, row);
        }
      }
    }
  }
}

// Compute operand type: bf16 for bf16 / fp8 pages, fp16 for NVFP4 pages.
template <int FMT> struct OpType { typedef bf16x8 type; };
template <> struct OpType<kFmtNvfp4> { typedef f16x8 type; };

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

// Decode V row i into NN half-precision values (packed pairs).
template <int FMT, int D>
__device__ __forceinline__ void v_row(const ChunkRaw<FMT, D>& raw, int i, uint32_t out[D / 32]) {
  constexpr int NN = D / 16;
  if constexpr (FMT == kFmtBf16) {
#pragma unroll
    for (int w = 0; w < NN / 2; ++w) out[w] = raw.v[i][w];
  } else if constexpr (FMT == kFmtFp8) {
#pragma unroll
    for (int w = 0; w < NN / 4; ++w) {
      out[2 * w] = fp8x2_to_bf16x2<false>(raw.v[i][w]);
      out[2 * w + 1] = fp8x2_to_bf16x2<true>(raw.v[i][w]);
    }
  } else {
    const f16x2 sc = fp8x2_to_f16x2<false>(raw.vs[i]);
    const f16x2 s = {sc[0], sc[0]};
    const uint32_t w = raw.v[i];
    out[0] = f16x2_bits(fp4x2_to_f16x2<0>(w) * s);
    out[1] = f16x2_bits(fp4x2_to_f16x2<1>(w) * s);
    out[2] = f16x2_bits(fp4x2_to_f16x2<2>(w) * s);
    out[3] = f16x2_bits(fp4x2_to_f16x2<3>(w) * s);
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

// One 32-token chunk of one wave.  The next chunk's K is loaded as soon as
// this chunk's QK^T products have consumed K, and its V once the V operands
// are built, so one set of staging registers suffices.
template <int FMT, int D>
__device__ __forceinline__ void process_chunk(WaveState<FMT, D>& st, ChunkRaw<FMT, D>& raw,
                                              const typename OpType<FMT>::type* qop, float sl2, int c, int ctx,
                                              bool chunk_ok, int lane, const AttendArgs& a, const int* slot_list,
                                              int c_next, bool more, int kvh) {
  constexpr int KK = D / 32, NN = D / 16;
  typedef typename OpType<FMT>::type OT;
  const int g = lane >> 4;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    s0 = mfma16(k_operand<FMT, D>(raw, 0, kk), qop[kk], s0);
    s1 = mfma16(k_operand<FMT, D>(raw, 1, kk), qop[kk], s1);
  }
  ChunkAddr nca;
  if (more) {
    nca = chunk_addr<FMT>(a, slot_list, c_next);
    load_k<FMT, D>(raw, a, nca, c_next, ctx, kvh, lane);
  }
  // online softmax over this chunk's 32 tokens
  const int tok0 = c * 32 + 4 * g;
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = (chunk_ok && tok0 + i < ctx) ? s0[i] : -INFINITY;
    sc[4 + i] = (chunk_ok && tok0 + 16 + i < ctx) ? s1[i] : -INFINITY;
  }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
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
  u32x4 pw, onesw;
  if constexpr (FMT == kFmtNvfp4) {
    pw = u32x4{pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]), pack_f16(p[6], p[7])};
    onesw = u32x4{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
  } else {
    pw = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
    onesw = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  }
  const OT pop = __builtin_bit_cast(OT, pw);
  // V rows -> transposed operands (V^T rows d = r * NN + nn, keys tau(8g + i))
  uint32_t rows[8][NN / 2];
#pragma unroll
  for (int i = 0; i < 8; ++i) v_row<FMT, D>(raw, i, rows[i]);
  OT vop[NN];
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) {
    u32x4 vw;
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const uint32_t a0 = rows[2 * pr][nn >> 1], a1 = rows[2 * pr + 1][nn >> 1];
      vw[pr] = (nn & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
    }
    vop[nn] = __builtin_bit_cast(OT, vw);
  }
  if (more) load_v<FMT, D>(raw, a, nca, c_next, ctx, kvh, lane);
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) st.acc[nn] = mfma16(vop[nn], pop, st.acc[nn]);
  st.lacc = mfma16(__builtin_bit_cast(OT, onesw), pop, st.lacc);
}

// Shared memory of one workgroup.
template <int D>
struct AttendSmem {
  int slot_list[kMaxTopK];
  int ctx;
  float m[4][16];
  float l[4][16];
  float o[4][16][D];
};

template <int FMT, int D, int MODE>
__global__ __launch_bounds__(256) void attend_rows_kernel(const AttendArgs a) {
  constexpr int KK = D / 32, NN = D / 16;
  typedef typename OpType<FMT>::type OT;
  __shared__ AttendSmem<D> sm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  int bid = blockIdx.x;
  const int split = bid % a.nsplit;
  bid /= a.nsplit;
  const int kvh = bid % a.num_kv_heads;
  const int row = bid / a.num_kv_heads;

  int req, abs_pos;
  if constexpr (MODE == kModeDecode) {
    decode_row_position(a.seq_lens, a.dql, row, &req, &abs_pos);
  } else {
    prefill_row_position(a.cu_seqlens_q, a.seq_lens, a.num_reqs, row, &req, &abs_pos);
  }
  if (wave == 0) {
    const RowSlots rs = compact_row(a.topk + (int64_t)row * a.topk_stride, a.topk_k,
                                    a.block_table + (int64_t)req * a.bt_stride, a.bt_cols, abs_pos, sm.slot_list);
    if (lane == 0) sm.ctx = rs.ctx;
  }
  __syncthreads();
  const int ctx = sm.ctx;
  const int nchunks = (ctx + 31) >> 5;
  const int c0 = (int)((int64_t)nchunks * split / a.nsplit);
  const int c1 = (int)((int64_t)nchunks * (split + 1) / a.nsplit);

  // Q operand: head kvh*G + r (zero for padded heads r >= G)
  const int G = a.group;
  OT qop[KK];
  {
    const bool ok = r < G;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                          ((int64_t)row * a.num_q_heads + kvh * G + (ok ? r : 0)) * D * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w = load_or_zero<u32x4>(ok, qrow + 2 * kappa<FMT, D>(kk, g));
      if constexpr (FMT == kFmtNvfp4) {
        w = u32x4{bf16x2_to_f16x2(w[0]), bf16x2_to_f16x2(w[1]), bf16x2_to_f16x2(w[2]), bf16x2_to_f16x2(w[3])};
      }
      qop[kk] = __builtin_bit_cast(OT, w);
    }
  }
  const float kscale = a.k_scale ? *a.k_scale : 1.f;
  const float sl2 = a.softmax_scale * kscale * kLog2e;

  WaveState<FMT, D> st;
#pragma unroll
  for (int nn = 0; nn < NN; ++nn) st.acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.lacc = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;

  ChunkRaw<FMT, D> raw;
  int c = c0 + wave;
  if (c < c1) {
    const ChunkAddr ca = chunk_addr<FMT>(a, sm.slot_list, c);
    load_k<FMT, D>(raw, a, ca, c, ctx, kvh, lane);
    load_v<FMT, D>(raw, a, ca, c, ctx, kvh, lane);
  }
  for (; c < c1; c += 4) {
    const bool ok = chunk_addr<FMT>(a, sm.slot_list, c).ok;
    process_chunk<FMT, D>(st, raw, qop, sl2, c, ctx, ok, lane, a, sm.slot_list, c + 4, c + 4 < c1, kvh);
  }

  // merge the four waves through LDS
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
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += 256) {
    const int h = idx / (D / 4), d = (idx % (D / 4)) * 4;
    float M = sm.m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm.m[w][h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
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

template <int FMT, int D, int MODE>
static hipError_t launch_fmt(const AttendArgs& a, int rows, hipStream_t stream) {
  const int64_t blocks = (int64_t)rows * a.num_kv_heads * a.nsplit;
  hipLaunchKernelGGL((attend_rows_kernel<FMT, D, MODE>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int pairs = rows * a.num_q_heads;
  const int per_block = 256 / (D / 4);
  hipLaunchKernelGGL((attend_merge_kernel<D>), dim3((unsigned)((pairs + per_block - 1) / per_block)), dim3(256), 0,
                     stream, a, pairs);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const AttendArgs& a, int fmt, int rows, hipStream_t stream) {
  if (a.head_dim == 128) {
    if (fmt == kFmtBf16) return launch_fmt<kFmtBf16, 128, MODE>(a, rows, stream);
    if (fmt == kFmtFp8) return launch_fmt<kFmtFp8, 128, MODE>(a, rows, stream);
    return launch_fmt<kFmtNvfp4, 128, MODE>(a, rows, stream);
  }
  if (fmt == kFmtBf16) return launch_fmt<kFmtBf16, 64, MODE>(a, rows, stream);
  return launch_fmt<kFmtFp8, 64, MODE>(a, rows, stream);
}

hipError_t launch_attend_rows(const AttendArgs& a, int fmt, int mode, int rows, hipStream_t stream) {
  if (mode == kModeDecode) return launch_mode<kModeDecode>(a, fmt, rows, stream);
  return launch_mode<kModePrefill>(a, fmt, rows, stream);
}

}  // namespace msa
