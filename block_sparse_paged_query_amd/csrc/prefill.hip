// Block-sparse ragged causal prefill on matrix cores.
//
// [FI] vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
//      MiniMaxM3SparseFlashInferImpl.forward (msa_sparse_attention: ragged
//      rows by cu_seqlens_q, causal, per-token top-k blocks).
// [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4,
//      MiniMaxM3SparseRocmNvfp4Impl / MetadataBuilder.build (each prefill
//      token's request and absolute position).
// [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa,
//      _write_sparse_block_table_row_from_values (the tokens a row sees).
//
// Work decomposition.  A workgroup (16 waves, four per SIMD) owns one kv head
// and QT consecutive query rows of one request (QT = 16 RT, RT = floor(16 / G)
// rows per matrix tile for G query heads per kv head: 16 rows at G >= 9, 256
// at G = 1; a tile's 16 - RT G spare columns stay masked).  Every query row picks its own
// blocks, so the workgroup first builds, per block of the request, the bit
// mask of its rows that selected it (and may see it causally), then walks
// the blocks some row selected in ascending order (a window of blocks at a
// time for long contexts).  Each such block's K and V (128 keys x D bf16)
// go once into LDS by direct-to-LDS buffer loads issued by waves 0-7 (a
// scalar descriptor per block, 32-bit lane offsets; each lane's LDS slot is
// fixed, so layouts are made by choosing which global chunk a lane fetches),
// double-buffered: K as [key][d] with 16-byte chunks XOR-swizzled by key, V
// as [d pair of 16-byte chunks][key] so that the transposing read
// ds_read_b64_tr_b16 (a lane receives one column of the 4 key rows its
// 16-lane group points at) yields the V^T operand with no bank conflict.
// The next block's copies are all issued when a block starts, into the other
// buffer, so they have the whole block's compute to land.  Every wave owns one
// matrix tile of 16 columns = (16 / G query rows) x (G heads) and runs QK^T and
// PV only when a row of its tile selected the block; the other rows of an
// active tile are masked.  One tile per wave keeps a wave within 128 VGPRs, so
// four waves share each SIMD: a SIMD's active tiles sit in different waves
// and overlap, instead of running one after the other inside a wave.  Each
// chunk's K and V operands are read from LDS just before use (the other
// waves cover the latency).  Every block ends at a workgroup barrier, so each
// wave sets its issue priority from the work it has left in the block, which
// keeps a SIMD's waves in step instead of leaving the youngest to finish
// alone.  In a row's own block, the 32-key chunks past the wave's last row
// are skipped.  Online softmax state stays in registers; the workgroup
// writes its rows' bf16 outputs at the end.
// Workgroups of one kv head share an XCD (blockIdx % Hkv), so K/V blocks
// re-read by neighbouring query tiles hit that XCD's L2.  At 4 to 8 query
// heads per kv head a tile holds 2 to 4 rows, and a small kernel run first
// (pf_group_kernel) groups each query tile's rows with alike selections, so
// that fewer tiles are active per block.
//
// fp8 and NVFP4 pages ([FI] forward folds the fp8 scales; [NV4] customize_spec
// for the two NVFP4 slots) take a staged path: the selected block's raw bytes
// (half or a quarter of bf16's) go into LDS and are converted exactly (fp8 ->
// bf16; e2m1 x E4M3 block scale -> fp16) into the same K / V layouts the
// bf16 path reads, so the matrix-core loop is shared.  Waves 0-7 copy and
// convert, so the other waves of each SIMD keep computing meanwhile.  fp8
// stages into two raw buffers and converts each block at its start; NVFP4 (a
// smaller raw block) keeps two compute-layout buffers and converts the next
// block while the current one computes, each wave converting the page it
// copied, at raised priority.  NVFP4
// computes in fp16 (the query is converted once), fp8 in bf16; the
// per-tensor scales fold into the softmax scale and the output as in the
// decode.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

constexpr int kPfWaves = 16;                // four per SIMD
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfTiles = 1;                 // matrix tiles per wave
constexpr int kPfCopyWaves = 8;             // waves that copy, stage and convert K/V blocks
constexpr int kPfCopyThreads = 64 * kPfCopyWaves;
// Row masks: a workgroup tile has QT = 16 RT rows (32 for 8 query heads per
// kv head, 80 for 3, 256 for 1), so a block's mask is MW = ceil(QT / 32)
// words; the block masks of a window of kPfWindow<MW> blocks are held at once
// (a request with more blocks is walked window by window).
template <int MW>
constexpr int kPfWindow = MW <= 2 ? 2048 : 4096 / MW;
// NVFP4 holds two compute-layout blocks (4 x 32 KB) and one raw block
// (18 KB): its window is what the rest of the 160 KB leaves for the tables
// (per block: MW mask words, a list entry and a physical id).
template <int MW>
constexpr int kPfWindowAhead = ((160 * 1024 - 4 * 32768 - 8 * 2 * 9 * 128 - 512) / (4 * MW + 6)) & ~63;
// one block of K (or V) in the compute layout: 128 keys x D bf16 / fp16
template <int D>
constexpr int kPfBlockBytes = kBlockTokens * 2 * D;
// raw bytes of one block (one kv head, K and V) in the staging buffers
template <int D>
constexpr int kPfFp8RawBytes = 2 * kBlockTokens * D;                  // [key][D] K, then [16-byte piece][key] V
constexpr int kPfNvfp4RawBytes = kPagesPerBlock * 2 * 9 * 128;       // per page: K slot, V slot (1152 B each)
template <int FMT, int D>
constexpr int kPfRawBytes = FMT == kFmtBf16 ? kPfBlockBytes<D> : (FMT == kFmtFp8 ? kPfFp8RawBytes<D> : kPfNvfp4RawBytes);
// compute operand type: bf16 for bf16 / fp8 pages, fp16 for NVFP4 pages
template <int FMT> struct PfOp { typedef bf16x8 type; };
template <> struct PfOp<kFmtNvfp4> { typedef f16x8 type; };
// PV operand type: fp16 wherever V is exact in fp16 (E4M3, e2m1 x E4M3), so
// the probabilities keep 11 significant bits; bf16 pages stay bf16
template <int FMT> struct PfPv { typedef f16x8 type; };
template <> struct PfPv<kFmtBf16> { typedef bf16x8 type; };

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// K row swizzle: 16-byte chunk c of key row k sits at chunk c ^ (k & (D/8 - 1)).
template <int D>
__device__ __forceinline__ int k_swz(int key) { return key & (D / 8 - 1); }

typedef short v4i16 __attribute__((ext_vector_type(4)));

// V layout: 16-byte slot ((lc / 2) * 128 + key) * 2 + lc % 2 holds chunk lc
// (d = 8 lc .. 8 lc + 7) of key.

// The copy of block `phys` (logical block `blk`), kv head kvh, into LDS
// (kb, vb), by waves 0-7: each copies one 16-token page of K and an eighth of V,
// D / 32 instructions of 1 KB for each side.  K instruction (wave, part)
// holds keys 16 wave + (64 / L) part + lane / L (L = D / 8 lanes per key
// row); V instruction v = wave * (D / 32) + part holds keys 32 (v % 4) +
// lane / 2 at d chunk 2 (v / 4) + lane % 2.  So every address is a per-block
// scalar base plus a small per-lane offset.  Keys at or past seq_len (only
// in a request's last block) are read from key 0 of the block instead
// (finite data that gets probability zero), so no NaN of an unwritten slot
// reaches the products.
template <int D>
__device__ __forceinline__ void pf_issue_block(lds_u8* kb, lds_u8* vb, const AttendArgs& a, int kvh, int phys,
                                               int blk, int seq_len) {
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kPfCopyWaves) return;
  constexpr int L = D / 8, KPI = 64 / L, PARTS = D / 32;
  // (block ids come from LDS: make their uniformity explicit so that the
  // bases below are scalar and only 32-bit lane offsets stay in registers)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));   // recompute the lane offsets here rather than keep them live across blocks
  phys = __builtin_amdgcn_readfirstlane(phys);
  blk = __builtin_amdgcn_readfirstlane(blk);
  const int64_t boff = (int64_t)phys * a.blk_units * a.sub_stride + (int64_t)kvh * a.head_stride;
  const int rs = a.row_stride;
  const int nkeys = seq_len - blk * kBlockTokens;     // keys of this block that exist (>= 1)
  const int kq = lane / L, kpc = lane % L;            // K: key 16 wave + KPI part + kq, 16-byte chunk kpc
  const int vq = lane >> 1, vodd = lane & 1;          // V: key 32 (v % 4) + vq, chunk 2 (v / 4) + vodd
  if (nkeys >= kBlockTokens && a.sub_stride < (int64_t(1) << 27)) {
    // scalar buffer descriptors over the wave's K page and the block's V
    // pages; lanes add 32-bit offsets (V: a scalar offset per instruction)
    const int vspan = (int)(7 * a.sub_stride) + kPageTokens * rs;
    const __amdgpu_buffer_rsrc_t kr_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.k_base + boff + wave * a.sub_stride), (short)0, kPageTokens * rs, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr_ =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v_base + boff), (short)0, vspan, kRawBufferWord3);
    const int voff = (vq >> 4) * (int)a.sub_stride + (vq & 15) * rs + (vodd << 4);
#pragma unroll
    for (int part = 0; part < PARTS; ++part) {
      const int kr = KPI * part + kq;                 // key within the wave's page
      const int koff = kr * rs + ((kpc ^ k_swz<D>(kr)) << 4);
      const int v = wave * PARTS + part;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr_, kb + (wave * PARTS + part) * 1024, 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr_, vb + v * 1024, 16, voff,
                                               2 * (v & 3) * (int)a.sub_stride + 32 * (v >> 2), 0, 0);
    }
  } else {
#pragma unroll
    for (int part = 0; part < PARTS; ++part) {
      const int v = wave * PARTS + part;
      const int kkey = 16 * wave + KPI * part + kq, vkey = 32 * (v & 3) + vq;
      const int ks = kkey < nkeys ? kkey : 0, vs = vkey < nkeys ? vkey : 0;
      const int kcol = (kpc ^ k_swz<D>(kkey)) << 4;
      __builtin_amdgcn_global_load_lds(a.k_base + boff + (ks >> 4) * a.sub_stride + (ks & 15) * rs + kcol,
                                       kb + (wave * PARTS + part) * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.v_base + boff + (vs >> 4) * a.sub_stride + (vs & 15) * rs +
                                           ((2 * (v >> 2) + vodd) << 4),
                                       vb + v * 1024, 16, 0, 0);
    }
  }
}

template <class OT, int D>
struct PfWave {
  static constexpr int KK = D / 32, NN = D / 16;
  OT qop[kPfTiles][KK];
  f32x4 acc[kPfTiles][NN];
  float lsum[kPfTiles];   // softmax denominators: this lane's share (its 8 keys of each chunk)
  float m[kPfTiles];
  int lrow[kPfTiles];     // row within the workgroup tile, or -1
  int lbit[kPfTiles];     // its bit in the wave's block mask
  int lpos[kPfTiles];     // that row's absolute position
  int last_pos;           // the wave's last row position (uniform), -1 without rows
};

// Online softmax keeps, per (row, head), a reference max m and rescales the
// accumulators only when some lane's chunk max exceeds m by more than kLazy
// (log2 units): probabilities are then at most 2^kLazy, well inside bf16 /
// fp32 range.  The common case needs no cross-lane max and no rescale.  Each
// lane sums the rounded probabilities it feeds the PV product (two per dot
// instruction), so the denominator sums exactly what the products use; the
// four lanes of a column are added at the end.
constexpr float kLazy = 8.f;

// acc + the two probabilities packed in w (a bf16 or fp16 pair)
template <class PT>
__device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
  if constexpr (__is_same(PT, f16x8)) {
    return __builtin_amdgcn_fdot2(bits_f16x2(w), bits_f16x2(0x3c003c00u), acc, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
  }
}

// One 32-key chunk against the tiles in MASK (a compile-time set, so that the
// phases below form straight-line code): all QK^T products, then all
// softmaxes (one uniform branch covers the rare rescale of any tile), then all
// PV products.  `read_v` reads this chunk's V operands once the QK^T products
// have consumed the K operands (into registers the K operands no longer
// need), so those LDS reads overlap the softmax.
template <int MASK, int D, class OT, class PT, class ReadV>
__device__ __forceinline__ void pf_chunk(PfWave<OT, D>& w, const OT (&kop)[2][PfWave<OT, D>::KK],
                                         PT (&vop)[PfWave<OT, D>::NN], const float (&bias)[kPfTiles], float sl2,
                                         bool causal, int kbase, ReadV&& read_v) {
  constexpr int KK = PfWave<OT, D>::KK, NN = PfWave<OT, D>::NN;
  constexpr bool kF16 = __is_same(PT, f16x8);
  float sv[kPfTiles][8];
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    if (!((MASK >> i) & 1)) continue;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mfma16(kop[0][kk], w.qop[i][kk], s0);
      s1 = mfma16(kop[1][kk], w.qop[i][kk], s1);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      sv[i][ii] = s0[ii];
      sv[i][4 + ii] = s1[ii];
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // the V reads must not rise above the products reading kop
  read_v(vop);
  float mxs[kPfTiles];
  bool need = false;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    if (!((MASK >> i) & 1)) continue;
    if (causal) {
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int kp = kbase + (ii & 3) + ((ii >> 2) << 4);
        sv[i][ii] = kp <= w.lpos[i] ? sv[i][ii] : -INFINITY;
      }
    }
    // (IEEE maximum: one v_maximum3 per two scores, no NaN-quieting moves;
    // a NaN score gives a NaN probability either way)
    float mx = sv[i][0];
#pragma unroll
    for (int ii = 1; ii < 8; ++ii) mx = __builtin_elementwise_maximum(mx, sv[i][ii]);
    mxs[i] = fmaf(mx, sl2, bias[i]);                       // this lane's chunk max, scaled (log2 units)
    need |= mxs[i] > w.m[i] + kLazy;
  }
  if (__ballot(need)) {                                    // rare after the first chunk of a row
#pragma unroll
    for (int i = 0; i < kPfTiles; ++i) {
      if (!((MASK >> i) & 1)) continue;
      float mh = fmaxf(mxs[i], __shfl_xor(mxs[i], 16));
      mh = fmaxf(mh, __shfl_xor(mh, 32));                  // the head's chunk max
      const float m_new = fmaxf(w.m[i], mh);
      const float alpha = exp2_fast(w.m[i] - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = w.acc[i][nn] * alpha;
      w.lsum[i] *= alpha;
      w.m[i] = m_new;
    }
  }
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    if (!((MASK >> i) & 1)) continue;
    const float off = bias[i] - (w.m[i] == -INFINITY ? 0.f : w.m[i]);
    float p[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) p[ii] = exp2_fast(fmaf(sv[i][ii], sl2, off));
    u32x4 pw;
    if constexpr (kF16) {
      pw = u32x4{pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]), pack_f16(p[6], p[7])};
    } else {
      pw = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
    }
    const PT pop = __builtin_bit_cast(PT, pw);
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = mfma16(vop[nn], pop, w.acc[i][nn]);
#pragma unroll
    for (int e = 0; e < 4; ++e) w.lsum[i] = dot2_ones<PT>(pw[e], w.lsum[i]);
  }
}

struct PfNext {       // the block whose copies are issued during this one
  lds_u8* kb;
  lds_u8* vb;
  int phys, blk;
  bool valid;
};

// The block's four 32-key chunks against the tiles in MASK.  Each chunk's K
// operands are read from LDS when the chunk starts and its V operands after
// its QK^T products; a wave holds one chunk's operands at a time, and the
// other waves of its SIMD cover the read latency.
template <int MASK, int D, class OT, class PT>
__device__ __forceinline__ void pf_chunks(PfWave<OT, D>& w, const uint8_t* kb, const uint8_t* vb,
                                          const int (&koff)[PfWave<OT, D>::KK], int voff,
                                          const float (&bias)[kPfTiles], float sl2, bool causal, int kbase0,
                                          int nch) {
  constexpr int KK = PfWave<OT, D>::KK, NN = PfWave<OT, D>::NN;
  auto load_k = [&](OT (&kop)[2][KK], int c) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[tt][kk] = *reinterpret_cast<const OT*>(kb + (c * 32 + 16 * tt) * (2 * D) + koff[kk]);
  };
  auto load_v = [&](PT (&vop)[NN], int c) {
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const v4i16 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (v4i16 __attribute__((address_space(3)))*)((const lds_u8*)vb + nn * 4096 + c * 1024 + voff));
      const v4i16 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (v4i16 __attribute__((address_space(3)))*)((const lds_u8*)vb + nn * 4096 + c * 1024 + 512 + voff));
      const u32x2 l0 = __builtin_bit_cast(u32x2, h0), l1 = __builtin_bit_cast(u32x2, h1);
      vop[nn] = __builtin_bit_cast(PT, u32x4{l0[0], l0[1], l1[0], l1[1]});
    }
  };
  OT kop[2][KK];
  PT vop[NN];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c >= nch) break;   // chunks past the wave's last row hold only masked keys
    // Issue priority from the work left in the block (3 in the first chunk, 0
    // in the last): a CU issues from its oldest waves first, which would let
    // them run ahead and leave the youngest to finish the block alone, with
    // nothing to hide its latency; the block's barrier waits for that one.
    if (c == 0) __builtin_amdgcn_s_setprio(3);
    else if (c == 1) __builtin_amdgcn_s_setprio(2);
    else if (c == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    load_k(kop, c);
    pf_chunk<MASK, D, OT, PT>(w, kop, vop, bias, sl2, causal, kbase0 + c * 32,
                              [&](PT (&v)[NN]) { load_v(v, c); });
  }
}

// One selected block against this wave's tiles.  `bmask` holds the wave's
// rows that selected the block (bit i * RT + k: row k of tile i).  `causal`
// is set when the block can be the own block of a row of this workgroup
// (keys past a row's position must be masked); earlier blocks need only the
// row selection.  Waves 0-7 first issue their pieces of the next block's
// copies, active or not.
template <int D, class OT, class PT>
__device__ __forceinline__ void pf_compute_block(PfWave<OT, D>& w, const uint8_t* kb, const uint8_t* vb,
                                                 uint32_t bmask, int blk, int RT, float sl2, bool causal,
                                                 const PfNext& nx, const AttendArgs& a, int kvh, int seq_len) {
  constexpr int KK = PfWave<OT, D>::KK;
  static_assert(kPfTiles == 1, "one matrix tile per wave");
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  // per-lane LDS offsets (chunk / tile / step parts are compile-time)
  int koff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = r * (2 * D) + (((4 * kk + g) ^ k_swz<D>(r)) << 4);
  // transposing read of lane (j, g): key 4g + j/4 (+16 hh) of the chunk, the
  // 8 bytes at d = 16 nn + 4 (j % 4)
  const int voff = g * 128 + (r >> 2) * 32 + (r & 3) * 8;
  // tiles of this wave that some row selected, and per-lane row selection:
  // bias 0 for a selected row, -inf otherwise
  float bias[kPfTiles];
  int tiles = 0;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    const uint32_t tile_bits = (uint32_t)((1ull << RT) - 1ull) << (i * RT);
    tiles |= (bmask & tile_bits) ? (1 << i) : 0;
    // (a slot without a row, or a spare column's bit past the tile, is never set)
    const bool sel = (bmask >> w.lbit[i]) & 1u;
    bias[i] = sel ? 0.f : -INFINITY;
  }
  const int kpos_blk = blk * kBlockTokens;
  if (nx.valid) pf_issue_block<D>(nx.kb, nx.vb, a, kvh, nx.phys, nx.blk, seq_len);
  // in a row's own block, the chunks past the wave's last row are masked for
  // all of the wave's rows
  const int nch = causal ? min(4, (w.last_pos - kpos_blk) / 32 + 1) : 4;
  if (tiles) pf_chunks<1, D, OT, PT>(w, kb, vb, koff, voff, bias, sl2, causal, kpos_blk + 4 * g, nch);
  __builtin_amdgcn_s_setprio(0);
}

// ---- staged formats -------------------------------------------------------
//
// Copy of one block's raw bytes (kv head kvh) into the staging buffer `raw`,
// spread over waves 0-7: each wave instruction fills 64 consecutive 16-byte
// slots, a lane's source being any 16-byte piece.
//   fp8:   K as [key][D B] (piece (key, n) at key * D / 16 + n), then V as
//          [n][key] (piece 8 D + n * 128 + key) so that the conversion
//          writes the V layout with consecutive lanes on consecutive keys.
//   NVFP4: the block's 8 pages, each the K slot then the V slot of kvh
//          (2 x 1152 B, adjacent in the page), piece q at q (head_dim 128).
//          Wave w copies page w (two full instructions and 16 lanes of a
//          third), so the wave that converts a page has copied it itself.
template <int FMT, int D>
__device__ __forceinline__ void pf_stage_issue(lds_u8* raw, const AttendArgs& a, int kvh, int phys) {
  constexpr int NPK = D / 16, HALF = kBlockTokens * NPK;   // pieces per key row; K pieces
  constexpr int kPfThreads = kPfCopyThreads;              // (the loops below run on waves 0-7)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= kPfCopyWaves) return;
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));   // recompute the lane offsets here rather than keep them live across blocks
  phys = __builtin_amdgcn_readfirstlane(phys);
  const int64_t boff = (int64_t)phys * a.blk_units * a.sub_stride + (int64_t)kvh * a.head_stride;
  if (a.sub_stride < (int64_t(1) << 27)) {
    // scalar buffer descriptors over the block's pages, 32-bit lane offsets
    const int sub = (int)a.sub_stride;
    if constexpr (FMT == kFmtFp8) {
      const int rs = a.row_stride, span = 7 * sub + kPageTokens * rs;
      const __amdgpu_buffer_rsrc_t kr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.k_base + boff),
                                                                           (short)0, span, kRawBufferWord3);
      const __amdgpu_buffer_rsrc_t vr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v_base + boff),
                                                                           (short)0, span, kRawBufferWord3);
#pragma unroll
      for (int k = 0; k < 2 * HALF / kPfThreads; ++k) {
        const int q = k * kPfThreads + wave * 64 + lane;
        const bool vs = k >= HALF / kPfThreads;
        const int key = vs ? (q - HALF) & 127 : q / NPK, n = vs ? (q - HALF) >> 7 : q % NPK;
        const int off = (key >> 4) * sub + (key & 15) * rs + 16 * n;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vs ? vr_ : kr_, raw + (k * kPfThreads + wave * 64) * 16, 16, off,
                                                 0, 0, 0);
      }
    } else {
      constexpr int PAGE = 2 * kNvfp4SlotBytes, TAIL = PAGE / 16 - 128;   // 2304 B; 16 pieces past 2 KB
      const __amdgpu_buffer_rsrc_t r_ = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.k_base + boff + (int64_t)wave * sub), (short)0, PAGE, kRawBufferWord3);
      lds_u8* dst = raw + wave * PAGE;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, dst, 16, 16 * lane, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, dst + 1024, 16, 1024 + 16 * lane, 0, 0, 0);
      if (lane < TAIL) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, dst + 2048, 16, 2048 + 16 * lane, 0, 0, 0);
    }
    return;
  }
  if constexpr (FMT == kFmtFp8) {
    const int rs = a.row_stride;
#pragma unroll
    for (int k = 0; k < 2 * HALF / kPfThreads; ++k) {
      const int q = k * kPfThreads + wave * 64 + lane;
      const uint8_t* src;
      if (k < HALF / kPfThreads) {
        const int key = q / NPK, n = q % NPK;
        src = a.k_base + boff + (key >> 4) * a.sub_stride + (key & 15) * rs + 16 * n;
      } else {
        const int q2 = q - HALF, n = q2 >> 7, key = q2 & 127;
        src = a.v_base + boff + (key >> 4) * a.sub_stride + (key & 15) * rs + 16 * n;
      }
      __builtin_amdgcn_global_load_lds(src, raw + (k * kPfThreads + wave * 64) * 16, 16, 0, 0);
    }
  } else {
    constexpr int PAGE = 2 * kNvfp4SlotBytes, TAIL = PAGE / 16 - 128;
    const uint8_t* src = a.k_base + boff + (int64_t)wave * a.sub_stride + 16 * lane;
    lds_u8* dst = raw + wave * PAGE;
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(src + 1024, dst + 1024, 16, 0, 0);
    if (lane < TAIL) __builtin_amdgcn_global_load_lds(src + 2048, dst + 2048, 16, 0, 0);
  }
}

// Exact conversion of a staged block into the compute layouts (K rows with
// 16-byte chunks swizzled by key; V as ((lc / 2) * 128 + key) * 2 + lc % 2):
// item (key, n) is the 16 elements d = 16 n .. 16 n + 15, i.e. chunks 2n and
// 2n + 1.  Keys at or past `nkeys` (the request's end, in its last block)
// become zeros, which the causal mask gives probability zero.
template <int FMT, int D>
__device__ __forceinline__ void pf_stage_item(const uint8_t* raw, bool v_side, int key, int n, uint32_t out[8]) {
  if constexpr (FMT == kFmtFp8) {
    // K -> bf16 (the QK^T operand type), V -> fp16 (the PV operand type)
    const u32x4 w =
        *reinterpret_cast<const u32x4*>(raw + (v_side ? kBlockTokens * D + (n * 128 + key) * 16 : key * D + 16 * n));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = v_side ? f16x2_bits(fp8x2_to_f16x2<false>(w[i])) : fp8x2_to_bf16x2<false>(w[i]);
      out[2 * i + 1] = v_side ? f16x2_bits(fp8x2_to_f16x2<true>(w[i])) : fp8x2_to_bf16x2<true>(w[i]);
    }
  } else {
    const uint8_t* slot = raw + (key >> 4) * (2 * kNvfp4SlotBytes) + (v_side ? kNvfp4SlotBytes : 0);
    const int tok = key & 15;
    // code bytes 8n .. 8n+7 (elements 16n .. 16n+15): two 4-byte units
    const u32x2 w = {*reinterpret_cast<const uint32_t*>(slot + nvfp4_code_byte(v_side, tok, 8 * n)),
                     *reinterpret_cast<const uint32_t*>(slot + nvfp4_code_byte(v_side, tok, 8 * n + 4))};
    const f16x2 sc = fp8x2_to_f16x2<false>((uint32_t)slot[nvfp4_scale_byte(v_side, tok, n)]);
    const f16x2 s2 = {sc[0], sc[0]};
    out[0] = f16x2_bits(fp4x2_to_f16x2<0>(w[0]) * s2);
    out[1] = f16x2_bits(fp4x2_to_f16x2<1>(w[0]) * s2);
    out[2] = f16x2_bits(fp4x2_to_f16x2<2>(w[0]) * s2);
    out[3] = f16x2_bits(fp4x2_to_f16x2<3>(w[0]) * s2);
    out[4] = f16x2_bits(fp4x2_to_f16x2<0>(w[1]) * s2);
    out[5] = f16x2_bits(fp4x2_to_f16x2<1>(w[1]) * s2);
    out[6] = f16x2_bits(fp4x2_to_f16x2<2>(w[1]) * s2);
    out[7] = f16x2_bits(fp4x2_to_f16x2<3>(w[1]) * s2);
  }
}

template <int FMT, int D>
__device__ __forceinline__ void pf_stage_convert(const uint8_t* raw, uint8_t* kc, uint8_t* vc, int nkeys) {
  constexpr int NPK = D / 16, HALF = kBlockTokens * NPK;
  constexpr int kPfThreads = kPfCopyThreads;              // waves 0-7 convert
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kPfCopyWaves) return;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));    // as in the copy issue: offsets recomputed per block
#pragma unroll
  for (int k = 0; k < 2 * HALF / kPfThreads; ++k) {
    const int q = k * kPfThreads + tid;
    const bool v_side = k >= HALF / kPfThreads;
    const int key = v_side ? ((q - HALF) & 127) : (q / NPK);
    const int n = v_side ? ((q - HALF) >> 7) : (q % NPK);
    uint32_t o[8];
    pf_stage_item<FMT, D>(raw, v_side, key, n, o);
    if (key >= nkeys) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = 0u;
    }
    const u32x4 c0 = {o[0], o[1], o[2], o[3]}, c1 = {o[4], o[5], o[6], o[7]};
    if (!v_side) {
      const int sw = k_swz<D>(key);   // chunk c of the key row sits at c ^ sw
      *reinterpret_cast<u32x4*>(kc + key * (2 * D) + (((2 * n) ^ sw) << 4)) = c0;
      *reinterpret_cast<u32x4*>(kc + key * (2 * D) + (((2 * n + 1) ^ sw) << 4)) = c1;
    } else {
      *reinterpret_cast<u32x4*>(vc + (n * 128 + key) * 32) = c0;
      *reinterpret_cast<u32x4*>(vc + (n * 128 + key) * 32 + 16) = c1;
    }
  }
}

// NVFP4, one quarter of the calling wave's own page: wave w converts the 16
// keys of page w (the page it copied), items q = 64 part + lane of 256: K
// items first (key 16 w + q / 8, piece q % 8), then V items (key 16 w +
// q % 16, piece (q - 128) / 16, consecutive lanes on consecutive keys).
template <int D>
__device__ __forceinline__ void pf_convert_own_page(const uint8_t* raw, uint8_t* kc, uint8_t* vc, int nkeys,
                                                    int part) {
  static_assert(D == 128, "NVFP4 pages hold head_dim 128");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= kPfCopyWaves) return;   // waves 0-7 copied the block's 8 pages
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const bool v_side = part >= 2;
  const int local = (64 * part + lane) & 127;
  const int key = 16 * wave + (v_side ? (local & 15) : (local >> 3));
  const int n = v_side ? (local >> 4) : (local & 7);
  uint32_t o[8];
  pf_stage_item<kFmtNvfp4, D>(raw, v_side, key, n, o);
  if (key >= nkeys) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0u;
  }
  const u32x4 c0 = {o[0], o[1], o[2], o[3]}, c1 = {o[4], o[5], o[6], o[7]};
  if (!v_side) {
    const int sw = k_swz<D>(key);
    *reinterpret_cast<u32x4*>(kc + key * (2 * D) + (((2 * n) ^ sw) << 4)) = c0;
    *reinterpret_cast<u32x4*>(kc + key * (2 * D) + (((2 * n + 1) ^ sw) << 4)) = c1;
  } else {
    *reinterpret_cast<u32x4*>(vc + (n * 128 + key) * 32) = c0;
    *reinterpret_cast<u32x4*>(vc + (n * 128 + key) * 32 + 16) = c1;
  }
}

// The query tile with index t, as every prefill kernel enumerates them:
// first ceil(rows / QT) tiles of each request in request order (mode 0),
// then padding tiles over rows [0, cu[0]) and [cu[R], total) (mode 1).
// Row ranges are clamped to [0, total_rows); an empty range means nothing
// to do.  Run by one whole wave; every lane gets the result.
struct PfTile {
  int mode, req, row0, row_end;
};

__device__ __forceinline__ PfTile pf_find_tile(const AttendArgs& a, int t, int QT, int lane) {
  const int R = a.num_reqs;
  int running = 0, found_req = -1, found_row0 = 0;
  for (int base = 0; base < R; base += 64) {
    const int rq = base + lane;
    const int n = rq < R ? (a.cu_seqlens_q[rq + 1] - a.cu_seqlens_q[rq] + QT - 1) / QT : 0;
    const int incl = wave_incl_scan(n, lane);
    const int excl = incl - n;
    const bool hit = rq < R && t >= running + excl && t < running + incl;
    const uint64_t hm = __ballot(hit);
    if (hm) {
      const int src = __ffsll((unsigned long long)hm) - 1;
      found_req = __shfl(rq, src);
      found_row0 = __shfl(rq < R ? a.cu_seqlens_q[rq] + (t - running - excl) * QT : 0, src);
    }
    running += __shfl(incl, 63);
  }
  // rows outside [cu[0], cu[R]) are padding; every range is clamped to
  // [0, total_rows), so offsets past the buffers are never formed
  const int total = a.total_rows;
  const int head_end = min(max(a.cu_seqlens_q[0], 0), total);
  const int real_end = min(max(a.cu_seqlens_q[R], head_end), total);
  PfTile tl;
  if (found_req >= 0) {
    tl.mode = 0;
    tl.req = found_req;
    tl.row0 = min(max(found_row0, 0), total);
    tl.row_end = min(min(found_row0 + QT, a.cu_seqlens_q[found_req + 1]), total);
  } else {
    // padding tiles follow the real ones: rows [0, cu[0]), then [cu[R], total)
    const int p = t - running, n_head = (head_end + QT - 1) / QT;
    tl.mode = 1;
    tl.req = 0;
    if (p < n_head) {
      tl.row0 = p * QT;
      tl.row_end = min((p + 1) * QT, head_end);
    } else {
      tl.row0 = real_end + (p - n_head) * QT;
      tl.row_end = min(real_end + (p - n_head + 1) * QT, total);
    }
  }
  return tl;
}

// ---- row grouping for tiles of 2 to 4 rows -------------------------------
//
// At 4 to 8 query heads per kv head a matrix tile holds RT = 2 to 4 query
// rows (QT = 16 RT per workgroup), and it runs a block's products when any
// of its rows selected the block.  Rows whose selections overlap therefore
// share tiles: one wave per query tile groups its rows greedily.  The lowest
// ungrouped row opens a group; the group then takes, RT - 1 times, the
// ungrouped row with the highest 6 |common blocks| - |its blocks| against the
// blocks the group holds so far (the lowest such row on ties), each row's
// selected blocks folded to 64 bits.  Each finished group goes to the SIMD
// (waves s, s + 4, s + 8, s + 12 share one) whose groups so far share the
// fewest blocks with it, counted per block with multiplicity, so that a
// block's products spread over the four SIMDs; the group takes that SIMD's
// next free wave.  Any order gives the same results up to rounding (a row's
// softmax state is its own); this only orders the work.  On C4's
// independent draws the pairs cut the active (tile, block) pairs by 7 % and
// the busiest SIMD's share of a block by 7 %.
constexpr bool pf_groups_rows(int RT) { return RT >= 2 && RT <= 4; }

// perm[RT w + k] = row k of the group on wave w, or -1.
__device__ __forceinline__ void pf_group_rows(const uint32_t (*sig_w)[2], int8_t* perm, int nrows, int RT) {
  const int lane = threadIdx.x & 63;
  const bool mine = lane < nrows;
  const uint32_t lo = mine ? sig_w[lane][0] : 0u, hi = mine ? sig_w[lane][1] : 0u;
  const uint64_t sig = ((uint64_t)hi << 32) | lo;
  const int base = 64 - __popcll(sig);   // scores 6 common + 64 - own count lie in [0, 448]
  uint64_t U = __ballot(mine);           // rows not yet in a group
  // lane q < 4 keeps SIMD q's per-block tile counts (0 to 4) as three bit planes
  uint64_t P0 = 0, P1 = 0, P2 = 0;
  int cap = 0;
  perm[lane] = (int8_t)-1;
  while (U) {
    int rows[4] = {__ffsll((unsigned long long)U) - 1, -1, -1, -1};
    U &= U - 1;
    uint64_t act = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, rows[0]) << 32) |
                   (uint32_t)__builtin_amdgcn_readlane(lo, rows[0]);
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      if (k >= RT || !U) break;
      const int sc = 6 * __popcll(act & sig) + base;
      uint64_t C = U;   // the best candidates so far, narrowed one score bit at a time
#pragma unroll
      for (int b = 8; b >= 0; --b) {
        const uint64_t B = __ballot((sc >> b) & 1) & C;
        if (B) C = B;
      }
      rows[k] = __ffsll((unsigned long long)C) - 1;
      U &= ~(1ull << rows[k]);
      act |= ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, rows[k]) << 32) |
             (uint32_t)__builtin_amdgcn_readlane(lo, rows[k]);
    }
    const int d = __popcll(P0 & act) + 2 * __popcll(P1 & act) + 4 * __popcll(P2 & act);
    const int key = lane < 4 && cap < 4 ? (d << 2) | lane : 0x7fffffff;
    const int best = min(min(__builtin_amdgcn_readlane(key, 0), __builtin_amdgcn_readlane(key, 1)),
                         min(__builtin_amdgcn_readlane(key, 2), __builtin_amdgcn_readlane(key, 3))) & 3;
    const int wv = best + 4 * __builtin_amdgcn_readlane(cap, best);
    if (lane == best) {
      const uint64_t c0 = P0 & act, c1 = P1 & c0;
      P0 ^= act;
      P1 ^= c0;
      P2 |= c1;
      ++cap;
    }
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < RT) perm[RT * wv + k] = (int8_t)rows[k];
    }
  }
}

// One workgroup per query tile t (the prefill kernel's numbering): its 512
// threads read the tile's top-k rows, wave 0 groups the rows and writes the
// tile's QT-slot row order to perm_out[QT t ..] for every real tile below cap
// (padding tiles have no order).
constexpr int kGroupThreads = 512;

__global__ __launch_bounds__(kGroupThreads) void pf_group_kernel(const AttendArgs a, int8_t* perm_out, int cap) {
  __shared__ uint32_t s_sig[64][2];
  __shared__ int8_t s_perm[64];
  __shared__ int s_tile[4];
  const int RT = 16 / a.group, QT = kPfWaves * kPfTiles * RT;
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (t >= cap) return;
  if (tid < 64) {
    const PfTile tl = pf_find_tile(a, t, QT, lane);
    if (tid == 0) {
      s_tile[0] = tl.mode;
      s_tile[1] = tl.req;
      s_tile[2] = tl.row0;
      s_tile[3] = tl.row_end;
    }
  }
  if (tid < 128) s_sig[tid >> 1][tid & 1] = 0u;
  __syncthreads();
  const int mode = s_tile[0], req = s_tile[1], row0 = s_tile[2], row_end = s_tile[3];
  if (mode != 0 || row0 >= row_end) return;
  const int nrows = row_end - row0;
  const int cu0 = a.cu_seqlens_q[req], cu1 = a.cu_seqlens_q[req + 1];
  const int pos_first = a.seq_lens[req] - (cu1 - cu0) + (row0 - cu0);
  const int pos_last = pos_first + nrows - 1;
  const int nblk = pos_last < 0 ? 0 : min(pos_last / kBlockTokens + 1, a.bt_cols);
  const bool group = nrows > 2 && nblk > 0;
  if (group) {
    for (int idx = tid; idx < nrows * a.topk_k; idx += kGroupThreads) {
      const int rr = idx / a.topk_k, tk = idx - rr * a.topk_k;
      const int pos = pos_first + rr;
      const int blk = a.topk[(int64_t)(row0 + rr) * a.topk_stride + tk];
      if (pos >= 0 && blk >= 0 && blk < nblk && blk <= pos / kBlockTokens)
        atomicOr(&s_sig[rr][(blk >> 5) & 1], 1u << (blk & 31));
    }
    __syncthreads();
  }
  if (tid >= 64) return;
  if (group) {
    pf_group_rows(s_sig, s_perm, nrows, RT);
  } else {
    s_perm[lane] = (int8_t)(lane < nrows ? lane : -1);
  }
  if (lane < QT) perm_out[(int64_t)t * QT + lane] = s_perm[lane];
}

template <int FMT, int D, int MW>
__global__ __launch_bounds__(kPfThreads) void prefill_blocks_kernel(const AttendArgs a, int n_slots) {
  typedef typename PfOp<FMT>::type OT;
  typedef typename PfPv<FMT>::type PT;
  // NVFP4 converts the next block while the current one computes (two
  // compute-layout buffers, one raw buffer); fp8 has no room for that
  constexpr bool kAhead = FMT == kFmtNvfp4;
  constexpr int KK = PfWave<OT, D>::KK, NN = PfWave<OT, D>::NN,
                WIN = kAhead ? kPfWindowAhead<MW> : kPfWindow<MW>;
  // Four LDS buffers as distinct objects: the loops below are unrolled by two,
  // so the compiler knows the in-flight copies target another buffer.
  //   bf16:        K / V double buffers (bA, bC) and (bB, bD)
  //   fp8 / NVFP4: compute K, V (bA, bB) and raw staging buffers bC, bD
  __shared__ __align__(16) uint8_t bA[kPfBlockBytes<D>], bB[kPfBlockBytes<D>];
  __shared__ __align__(16) uint8_t bC[kAhead ? kPfBlockBytes<D> : kPfRawBytes<FMT, D>];
  __shared__ __align__(16) uint8_t bD[kAhead ? kPfBlockBytes<D> : kPfRawBytes<FMT, D>];
  __shared__ __align__(16) uint8_t bE[kAhead ? kPfRawBytes<FMT, D> : 16];
  __shared__ uint32_t s_mask[WIN][MW];        // per block of the window: its selecting rows
  __shared__ uint16_t s_list[WIN];            // selected blocks of the window, ascending
  __shared__ int32_t s_phys[WIN];             // their physical block ids
  __shared__ int s_info[4];
  __shared__ int8_t s_perm[64];               // tiles of 2-4 rows: tile slot -> row
  __shared__ int8_t s_slot[64];               // tiles of 2-4 rows: row -> tile slot
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int G = a.group, RT = 16 / G, QT = kPfWaves * kPfTiles * RT;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int t = n_slots - 1 - (int)(blockIdx.x / a.num_kv_heads);   // heavy (late) tiles first

  // ---- which rows: a tile of one request, padding rows, or nothing.  The
  // tile's row order (two-row tiles) is read meanwhile, if there is one.
  const bool grouped = pf_groups_rows(RT);
  const bool have_perm = grouped && a.row_perm != nullptr && t < a.perm_cap;
  int perm_v = -1;
  if (have_perm && wave == 1 && lane < QT) perm_v = a.row_perm[(int64_t)t * QT + lane];
  if (wave == 0) {
    const PfTile tl = pf_find_tile(a, t, QT, lane);
    if (lane == 0) {
      s_info[0] = tl.mode;
      s_info[1] = tl.req;
      s_info[2] = tl.row0;
      s_info[3] = tl.row_end;
    }
  }
  __syncthreads();
  const int mode = s_info[0], req = s_info[1], row0 = s_info[2], row_end = s_info[3];
  if (row0 >= row_end) return;   // uniform: nothing to do
  if (mode == 1) {
    // padding rows attend nothing: zero their heads of this kv head
    const int per_row = G * D / 8;   // 16-byte stores
    for (int idx = tid; idx < (row_end - row0) * per_row; idx += kPfThreads) {
      const int rr = idx / per_row, wd = idx % per_row;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.out) +
                     (((int64_t)(row0 + rr) * a.num_q_heads + kvh * G) * D) * 2 + wd * 16;
      *reinterpret_cast<u32x4*>(dst) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const int cu0 = a.cu_seqlens_q[req], cu1 = a.cu_seqlens_q[req + 1];
  const int seq_len = a.seq_lens[req];
  const int ctx0 = seq_len - (cu1 - cu0);          // context before the new tokens
  const int pos_first = ctx0 + (row0 - cu0);
  const int pos_last = ctx0 + (row_end - 1 - cu0);
  const int nblk = pos_last < 0 ? 0 : min(pos_last / kBlockTokens + 1, a.bt_cols);
  const int32_t* bt_row = a.block_table + (int64_t)req * a.bt_stride;
  const int nrows = row_end - row0;
  // tiles of 2-4 rows: slot k of wave w holds row s_perm[RT w + k] (the
  // order pf_group_kernel chose, else the natural one); s_slot is the inverse
  if (grouped) {
    if (wave == 1 && lane < QT) {
      int p = have_perm ? perm_v : lane;
      if (p < 0 || p >= nrows) p = -1;
      s_perm[lane] = (int8_t)p;
      s_slot[lane] = (int8_t)-1;
      if (p >= 0) s_slot[p] = (int8_t)lane;
    }
    __syncthreads();
  }

  // ---- this wave's query operands and row data.  The wave's tile slots are
  // bits [wbit0, wbit0 + RT) of a block's mask; slot k holds row wbit0 + k,
  // or, in tiles of 2-4 rows, row s_perm[wbit0 + k].
  PfWave<OT, D> w;
  const int wbit0 = wave * kPfTiles * RT;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    const int slot = (wave * kPfTiles + i) * RT + r / G;
    int rr = slot < nrows ? slot : -1;
    if (grouped) rr = s_perm[slot & 63];
    const bool ok = r < RT * G && rr >= 0;
    w.lrow[i] = ok ? rr : -1;
    w.lbit[i] = slot - wbit0;
    w.lpos[i] = pos_first + (ok ? rr : 0);
    w.m[i] = -INFINITY;
    w.lsum[i] = 0.f;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                          (((int64_t)(row0 + (ok ? rr : 0)) * a.num_q_heads + kvh * G + (r % G)) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 q4 = ok ? *reinterpret_cast<const u32x4*>(qrow + 2 * (32 * kk + 8 * g)) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (FMT == kFmtNvfp4) {
        q4 = u32x4{bf16x2_to_f16x2(q4[0]), bf16x2_to_f16x2(q4[1]), bf16x2_to_f16x2(q4[2]), bf16x2_to_f16x2(q4[3])};
      }
      w.qop[i][kk] = __builtin_bit_cast(OT, q4);
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  {
    int lp = w.lrow[0] >= 0 ? w.lpos[0] : -1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) lp = max(lp, __shfl_xor(lp, o));
    w.last_pos = __builtin_amdgcn_readfirstlane(lp);
  }
  const float kscale = a.k_scale ? *a.k_scale : 1.f;
  const float sl2 = a.softmax_scale * kscale * kLog2e;
  const int wword = wbit0 >> 5, wshift = wbit0 & 31;
  const uint32_t wave_bits = (uint32_t)((1ull << (kPfTiles * RT)) - 1ull);
  const int own_first = pos_first / kBlockTokens;   // blocks before it are wholly in every row's past

  // ---- the request's blocks, a window of WIN at a time (one window unless
  // the rows reach past WIN blocks); the softmax state carries across windows
  for (int w0 = 0; w0 < nblk; w0 += WIN) {
    const int w1 = min(w0 + WIN, nblk);
    if (w0 > 0) __syncthreads();   // every wave is done with the previous window's tables and buffers
    // per-block masks of the rows that selected the block (and may see it)
    for (int jj = tid; jj < (w1 - w0) * MW; jj += kPfThreads) s_mask[jj / MW][jj % MW] = 0u;
    __syncthreads();
    for (int idx = tid; idx < nrows * a.topk_k; idx += kPfThreads) {
      const int rr = idx / a.topk_k, tk = idx - rr * a.topk_k;
      const int pos = pos_first + rr;
      const int blk = a.topk[(int64_t)(row0 + rr) * a.topk_stride + tk];
      if (pos >= 0 && blk >= w0 && blk < w1 && blk <= pos / kBlockTokens)
      {
        const int sl = grouped ? (int)s_slot[rr] : rr;
        if (sl >= 0) atomicOr(&s_mask[blk - w0][sl >> 5], 1u << (sl & 31));
      }
    }
    __syncthreads();
    // selected blocks, ascending (blocks whose pages lie outside the cache are skipped)
    if (wave == 0) {
      int n = 0;
      for (int base = w0; base < w1; base += 64) {
        const int j = base + lane;
        bool act = false;
        if (j < w1) {
#pragma unroll
          for (int mw = 0; mw < MW; ++mw) act |= s_mask[j - w0][mw] != 0u;
        }
        if (act) {
          const int phys = bt_row[j];
          const int64_t last = (int64_t)phys * a.blk_units + a.v_unit_offset + kPagesPerBlock - 1;
          act = phys >= 0 && last < a.num_units;
        }
        const uint64_t am = __ballot(act);
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(am >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)am, 0u));
        if (act) {
          s_list[n + rank] = (uint16_t)(j - w0);
          s_phys[n + rank] = bt_row[j];
        }
        n += __popcll(am);
      }
      if (lane == 0) s_info[0] = n;
    }
    __syncthreads();
    const int n_act = s_info[0];
    // (readfirstlane returns int: shift the words as unsigned, or a set top
    // bit would smear into the bits of the next word)
    auto wave_mask = [&](int jl) -> uint32_t {
      uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane(s_mask[jl][wword]) >> wshift;
      if constexpr (MW > 1) {
        // a wave's RT bits run into the next word when RT does not divide 32
        if (wshift + kPfTiles * RT > 32)
          m |= (uint32_t)__builtin_amdgcn_readfirstlane(s_mask[jl][wword + 1]) << (32 - wshift);
      }
      return m & wave_bits;
    };

    if constexpr (FMT == kFmtBf16) {
      lds_u8 *k0 = (lds_u8*)bA, *k1 = (lds_u8*)bB, *v0 = (lds_u8*)bC, *v1 = (lds_u8*)bD;
      if (n_act > 0) {
        pf_issue_block<D>(k0, v0, a, kvh, s_phys[0], w0 + s_list[0], seq_len);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      for (int it = 0; it < n_act; it += 2) {
        // even step: block in (k0, v0); the next one goes to (k1, v1)
        {
          const int jl = s_list[it], j = w0 + jl;
          const PfNext nx = {k1, v1, it + 1 < n_act ? s_phys[it + 1] : 0,
                             it + 1 < n_act ? w0 + (int)s_list[it + 1] : 0, it + 1 < n_act};
          pf_compute_block<D, OT, PT>(w, bA, bC, wave_mask(jl), j, RT, sl2, j >= own_first, nx, a, kvh, seq_len);
          __builtin_amdgcn_s_waitcnt(0);   // this lane's copies of the next block have landed
          __syncthreads();
        }
        if (it + 1 >= n_act) break;
        // odd step: block in (k1, v1); the next one goes to (k0, v0)
        {
          const int jl = s_list[it + 1], j = w0 + jl;
          const PfNext nx = {k0, v0, it + 2 < n_act ? s_phys[it + 2] : 0,
                             it + 2 < n_act ? w0 + (int)s_list[it + 2] : 0, it + 2 < n_act};
          pf_compute_block<D, OT, PT>(w, bB, bD, wave_mask(jl), j, RT, sl2, j >= own_first, nx, a, kvh, seq_len);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
        }
      }
    } else if constexpr (kAhead) {
      // NVFP4: raw block in bE; each wave copies and converts its own page
      // (no barrier between the two), into (bA, bB) or (bC, bD).  The step
      // that computes block i first converts block i+1 into the other
      // compute buffers and issues block i+2's copy: one barrier per block.
      const PfNext none = {nullptr, nullptr, 0, 0, false};
      auto convert = [&](int idx, uint8_t* kc, uint8_t* vc) {
        // the next block's conversion goes ahead of the other waves' chunks
        // (the chunks then set their own priority)
        __builtin_amdgcn_s_setprio(3);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's copy of its page has landed
        const int nk = seq_len - (w0 + (int)s_list[idx]) * kBlockTokens;
#pragma unroll
        for (int part = 0; part < 4; ++part) pf_convert_own_page<D>(bE, kc, vc, nk, part);
      };
      if (n_act > 0) {
        pf_stage_issue<FMT, D>((lds_u8*)bE, a, kvh, s_phys[0]);
        convert(0, bA, bB);
        if (n_act > 1) pf_stage_issue<FMT, D>((lds_u8*)bE, a, kvh, s_phys[1]);
      }
      __syncthreads();
      for (int it = 0; it < n_act; it += 2) {
        {
          const int jl = s_list[it], j = w0 + jl;
          if (it + 1 < n_act) {
            convert(it + 1, bC, bD);
            if (it + 2 < n_act) pf_stage_issue<FMT, D>((lds_u8*)bE, a, kvh, s_phys[it + 2]);
          }
          pf_compute_block<D, OT, PT>(w, bA, bB, wave_mask(jl), j, RT, sl2, j >= own_first, none, a, kvh, seq_len);
          __syncthreads();   // every wave is done with (bA, bB), and (bC, bD) holds block it + 1
        }
        if (it + 1 >= n_act) break;
        {
          const int jl = s_list[it + 1], j = w0 + jl;
          if (it + 2 < n_act) {
            convert(it + 2, bA, bB);
            if (it + 3 < n_act) pf_stage_issue<FMT, D>((lds_u8*)bE, a, kvh, s_phys[it + 3]);
          }
          pf_compute_block<D, OT, PT>(w, bC, bD, wave_mask(jl), j, RT, sl2, j >= own_first, none, a, kvh, seq_len);
          __syncthreads();
        }
      }
    } else {
      // staged: raw block in bC / bD (alternating), converted into (bA, bB)
      const PfNext none = {nullptr, nullptr, 0, 0, false};
      if (n_act > 0) pf_stage_issue<FMT, D>((lds_u8*)bC, a, kvh, s_phys[0]);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      for (int it = 0; it < n_act; it += 2) {
        {
          const int jl = s_list[it], j = w0 + jl;
          pf_stage_convert<FMT, D>(bC, bA, bB, seq_len - j * kBlockTokens);
          __syncthreads();
          if (it + 1 < n_act) pf_stage_issue<FMT, D>((lds_u8*)bD, a, kvh, s_phys[it + 1]);
          pf_compute_block<D, OT, PT>(w, bA, bB, wave_mask(jl), j, RT, sl2, j >= own_first, none, a, kvh, seq_len);
          __builtin_amdgcn_s_waitcnt(0);   // this lane's copies of the next block have landed
          __syncthreads();                 // and every wave is done with (bA, bB)
        }
        if (it + 1 >= n_act) break;
        {
          const int jl = s_list[it + 1], j = w0 + jl;
          pf_stage_convert<FMT, D>(bD, bA, bB, seq_len - j * kBlockTokens);
          __syncthreads();
          if (it + 2 < n_act) pf_stage_issue<FMT, D>((lds_u8*)bC, a, kvh, s_phys[it + 2]);
          pf_compute_block<D, OT, PT>(w, bA, bB, wave_mask(jl), j, RT, sl2, j >= own_first, none, a, kvh, seq_len);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
        }
      }
    }
  }

  // ---- outputs: lane holds head r % G of row lrow, d = 16 nn + 4 g + ii
  const float vscale = a.v_scale ? *a.v_scale : 1.f;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    // the head's denominator: the four lanes of its column hold a quarter of the keys each
    float L = w.lsum[i];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (w.lrow[i] < 0) continue;
    const float inv = L > 0.f ? vscale / L : 0.f;
    uint8_t* orow = reinterpret_cast<uint8_t*>(a.out) +
                    (((int64_t)(row0 + w.lrow[i]) * a.num_q_heads + kvh * G + (r % G)) * D) * 2;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int d = 16 * nn + 4 * g;
      const u32x2 o = {pack_bf16(w.acc[i][nn][0] * inv, w.acc[i][nn][1] * inv),
                       pack_bf16(w.acc[i][nn][2] * inv, w.acc[i][nn][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d * 2) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Test hook: each row's K and V in sparse-table order, exactly as the prefill
// attend stages them.  One workgroup per (row, kv head, slot): the slot's
// block goes into LDS through the attend's own copy (pf_issue_block for bf16
// pages, pf_stage_issue for fp8 / NVFP4), and each (key, 16-element piece) is
// read back in the compute types: bf16 keys and values as copied, staged
// formats through pf_stage_item.  Values are the operand elements times
// k_scale / v_scale in fp32; keys at or past the row's context in the slot,
// and blocks outside the cache, give 0.  out[row][token][kv head][d].
// ---------------------------------------------------------------------------
template <int FMT, int D>
__global__ __launch_bounds__(kPfThreads) void gather_dequant_prefill_kernel(const AttendArgs a,
                                                                            const int32_t* __restrict__ sbt,
                                                                            int64_t sbt_stride,
                                                                            const int32_t* __restrict__ sctx, int bps,
                                                                            int width_tokens, float* __restrict__ k_out,
                                                                            float* __restrict__ v_out) {
  constexpr int NPK = D / 16;   // 16-element pieces of a key row
  __shared__ __align__(16) uint8_t bK[FMT == kFmtBf16 ? kPfBlockBytes<D> : 16];
  __shared__ __align__(16) uint8_t bV[FMT == kFmtBf16 ? kPfBlockBytes<D> : kPfRawBytes<FMT, D>];
  const int tid = threadIdx.x;
  const int nslot = width_tokens / kBlockTokens;
  const int slot = blockIdx.x % nslot;
  const int kvh = (blockIdx.x / nslot) % a.num_kv_heads;
  const int64_t row = blockIdx.x / nslot / a.num_kv_heads;
  const int ctx = min(max(sctx[row], 0), width_tokens);
  const int nkeys = min(ctx - slot * kBlockTokens, kBlockTokens);   // <= 0: slot past the context
  int phys = nkeys > 0 ? sbt[row * sbt_stride + kPagesPerBlock * slot] / bps : -1;
  const bool inside = phys >= 0 && (int64_t)phys * a.blk_units + a.v_unit_offset + kPagesPerBlock - 1 < a.num_units;
  const float ks = a.k_scale ? *a.k_scale : 1.f, vs = a.v_scale ? *a.v_scale : 1.f;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;
  float* kb = k_out + ((row * width_tokens + slot * kBlockTokens) * a.num_kv_heads + kvh) * D;
  float* vb = v_out + ((row * width_tokens + slot * kBlockTokens) * a.num_kv_heads + kvh) * D;
  if (inside) {   // uniform
    if constexpr (FMT == kFmtBf16) {
      pf_issue_block<D>((lds_u8*)bK, (lds_u8*)bV, a, kvh, phys, 0, nkeys);
    } else {
      pf_stage_issue<FMT, D>((lds_u8*)bV, a, kvh, phys);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  // item q: side q / (128 NPK), key, 16-element piece n (d = 16 n .. 16 n + 15)
  for (int q = tid; q < 2 * kBlockTokens * NPK; q += kPfThreads) {
    const bool v_side = q >= kBlockTokens * NPK;
    const int key = (q / NPK) & (kBlockTokens - 1), n = q % NPK;
    uint32_t o[8];
    if constexpr (FMT == kFmtBf16) {
      // K rows (2 D bytes): 16-byte chunk c of key at chunk c ^ k_swz(key);
      // V: chunk lc of key in the 16-byte slot ((lc / 2) * 128 + key) * 2 + lc % 2
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * n + h;
        const uint8_t* src = v_side ? bV + (((c >> 1) * kBlockTokens + key) * 2 + (c & 1)) * 16
                                    : bK + key * (2 * D) + ((c ^ k_swz<D>(key)) << 4);
        const u32x4 w = *reinterpret_cast<const u32x4*>(src);
        o[4 * h + 0] = w[0];
        o[4 * h + 1] = w[1];
        o[4 * h + 2] = w[2];
        o[4 * h + 3] = w[3];
      }
    } else {
      pf_stage_item<FMT, D>(bV, v_side, key, n, o);
    }
    const bool keep = inside && key < nkeys;
    float* dst = (v_side ? vb : kb) + (int64_t)key * tok_stride + 16 * n;
    const float sc = v_side ? vs : ks;
    // element types: bf16 pages bf16; fp8 K bf16, V fp16; NVFP4 fp16
    const bool as_f16 = FMT == kFmtNvfp4 || (FMT == kFmtFp8 && v_side);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float lo, hi;
      if (as_f16) {
        const f16x2 p = bits_f16x2(o[i]);
        lo = (float)p[0];
        hi = (float)p[1];
      } else {
        lo = __uint_as_float(o[i] << 16);
        hi = __uint_as_float(o[i] & 0xffff0000u);
      }
      dst[2 * i] = keep ? lo * sc : 0.f;
      dst[2 * i + 1] = keep ? hi * sc : 0.f;
    }
  }
}

hipError_t launch_gather_dequant_prefill(const AttendArgs& a, int fmt, const int32_t* sbt, int64_t sbt_stride,
                                         const int32_t* sctx, int bps, int rows, int width_tokens, float* k_out,
                                         float* v_out, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)rows * a.num_kv_heads * (width_tokens / kBlockTokens))), block(kPfThreads);
  log_launch("gather_dequant_prefill_kernel head_dim %d: %d rows x %d kv heads x %d blocks", a.head_dim, rows,
             a.num_kv_heads, width_tokens / kBlockTokens);
#define MSA_GATHER_PF(F, DD)                                                                                       \
  hipLaunchKernelGGL((gather_dequant_prefill_kernel<F, DD>), grid, block, 0, stream, a, sbt, sbt_stride, sctx, bps, \
                     width_tokens, k_out, v_out)
  if (a.head_dim == 128) {
    if (fmt == kFmtBf16) MSA_GATHER_PF(kFmtBf16, 128);
    else if (fmt == kFmtFp8) MSA_GATHER_PF(kFmtFp8, 128);
    else MSA_GATHER_PF(kFmtNvfp4, 128);
  } else {
    if (fmt == kFmtBf16) MSA_GATHER_PF(kFmtBf16, 64);
    else MSA_GATHER_PF(kFmtFp8, 64);
  }
#undef MSA_GATHER_PF
  return hipGetLastError();
}

// Row-mask words per block: ceil(16 RT / 32) for RT = floor(16 / G) rows per
// tile, so 8 at G = 1, 4 at 2, 3 at 3, 2 at 4 and 5, 1 from 6 up.
static int pf_mask_words(int group) { return (16 / group + 1) / 2; }

template <int FMT, int D>
static hipError_t launch_pf(const AttendArgs& a, dim3 grid, int n_slots, hipStream_t stream) {
  switch (pf_mask_words(a.group)) {
    case 1: hipLaunchKernelGGL((prefill_blocks_kernel<FMT, D, 1>), grid, dim3(kPfThreads), 0, stream, a, n_slots); break;
    case 2: hipLaunchKernelGGL((prefill_blocks_kernel<FMT, D, 2>), grid, dim3(kPfThreads), 0, stream, a, n_slots); break;
    case 3: hipLaunchKernelGGL((prefill_blocks_kernel<FMT, D, 3>), grid, dim3(kPfThreads), 0, stream, a, n_slots); break;
    case 4: hipLaunchKernelGGL((prefill_blocks_kernel<FMT, D, 4>), grid, dim3(kPfThreads), 0, stream, a, n_slots); break;
    default: hipLaunchKernelGGL((prefill_blocks_kernel<FMT, D, 8>), grid, dim3(kPfThreads), 0, stream, a, n_slots);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_blocks(const AttendArgs& a, int fmt, hipStream_t stream) {
  const int RT = 16 / a.group, QT = kPfWaves * kPfTiles * RT;
  // tiles: ceil(rows / QT) per request and per padding range (before the
  // first request, after the last) is at most ceil(total / QT) + R + 2
  const int n_slots = (a.total_rows + QT - 1) / QT + a.num_reqs + 2;
  const dim3 grid((unsigned)((int64_t)n_slots * a.num_kv_heads));
  // the caller's workspace (perm_cap units of 32 bytes) holds QT bytes of row
  // order per query tile; from here on perm_cap counts tiles
  AttendArgs ag = a;
  if (!pf_groups_rows(RT) || ag.row_perm == nullptr || (int64_t)ag.perm_cap * 32 < QT) {
    ag.row_perm = nullptr;
    ag.perm_cap = 0;
  } else {
    ag.perm_cap = (int32_t)((int64_t)ag.perm_cap * 32 / QT);
    const int n_group = min(n_slots, ag.perm_cap);
    log_launch("pf_group_kernel: %d query tiles of %d rows in groups of %d", n_group, QT, RT);
    hipLaunchKernelGGL(pf_group_kernel, dim3((unsigned)n_group), dim3(kGroupThreads), 0, stream, ag, ag.row_perm, n_group);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  log_launch("prefill_blocks_kernel %s pages, head_dim %d, %d query heads per kv head: %d tiles of %d rows x %d kv "
             "heads, 16 waves each", fmt == kFmtBf16 ? "bf16" : (fmt == kFmtFp8 ? "fp8" : "nvfp4"), a.head_dim,
             a.group, n_slots, QT, a.num_kv_heads);
  if (a.head_dim == 128) {
    if (fmt == kFmtBf16) return launch_pf<kFmtBf16, 128>(ag, grid, n_slots, stream);
    if (fmt == kFmtFp8) return launch_pf<kFmtFp8, 128>(ag, grid, n_slots, stream);
    return launch_pf<kFmtNvfp4, 128>(ag, grid, n_slots, stream);
  }
  if (fmt == kFmtBf16) return launch_pf<kFmtBf16, 64>(ag, grid, n_slots, stream);
  return launch_pf<kFmtFp8, 64>(ag, grid, n_slots, stream);
}

}  // namespace msa
