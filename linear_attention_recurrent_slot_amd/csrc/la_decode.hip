// la_decode.hip -- gfx950 kernels and C-ABI entry points for pool-indexed
// recurrent-state decode of linear attention (Lightning, GDN, KDA).
//
// The operation, argument layouts and error behaviour are specified in
// include/la_decode.h. The sources it follows:
//  - cuLA "fix: wire h0_indices into Lightning Attention decode for
//    state-pool indexing", Description: state read/written through the
//    request's slot index; grid over the active (request, head) units.
//  - FlashInfer "fp32 sibling of #3268", Description and "API change": 4D
//    pool [pool_size, HV, V, K] addressed in place through its strides,
//    separate write slots (negative = skip), multi-token verify with
//    optional per-token state caching.
//  - aiter "Fused Gluon KDA decode path (950/1250)", advisory review: the
//    per-token update (decay by exp(g), delta correction, output S^T q with
//    the updated state) with l2norm, sigmoid and gate fused into the kernel.
//
// Kernel design (gfx950, wave64):
//  - One workgroup per (request, value head) pair; V/R waves, each owning
//    R (32 by default) rows of the V x K fp32 state tile for the whole call. The tile is
//    held in VGPRs across all T tokens, so the pool sees one read and at most
//    one write per pair per call.
//  - Within a wave, 8 lanes share one row: lane (c, r) with c = lane & 7 and
//    r = lane >> 3 holds rows {R w + 8 i + r} and the 16-byte chunks
//    {c + 8 j} of each (4 fp32 or 8 bf16 columns). Each 128-bit buffer load
//    of the wave reads 8 whole 128-byte row segments; every byte of the tile
//    is read once and written once. Instances that write only the final
//    fp32 128 x 128 state pass it through a per-wave LDS area first, so each
//    store instruction covers 2 whole rows.
//  - Row dot products (S k and S q) reduce over the 8 lanes of a row with
//    three DPP butterfly adds; the butterfly leaves a bit-identical sum in
//    all 8 lanes, so the rank-1 update needs no broadcast.
//  - The per-token prologue (l2norm of q and k, beta sigmoid, exp of the
//    gate, the k.q product, v) is computed once per workgroup for up to 8
//    tokens at a time (2 when each token's state is written, 4 for KDA
//    calls of more than 4 tokens), one token per wave, and staged in LDS.
//  - Instances: 32 rows per wave; 16 on grids that fill less than one
//    resident round and with update records.
//  - Workgroups take their pairs in XCD blocks (xcd_block_pair): whole
//    requests per XCD below 48 value heads, 32-pair blocks from 48, the
//    plain order for dense KDA calls of more than four tokens without
//    per-token writes; the split one-token kernel deals blocks of four
//    whole tiles to the XCDs in turn.
//  - No MFMA: per token the work is two matrix-vector products and a rank-1
//    update against one vector operand, bound by HBM traffic of the state.
//  - Per token and element: one multiply (decay), two FMAs (read-outs) and
//    one FMA (update); Lightning needs no key read-out.
//  - Three kernels compute this: decode_kernel (the general one, which
//    serves every call), the packed one-token kernel for bf16 pools up to
//    2048 tiles (1536 for KDA) and the contiguous-row one-token kernel for
//    larger grids (decode1_kernel: each load instruction reads 1 KiB of
//    contiguous tile bytes, a wave owns 8 rows, and a 128 x 128 tile runs as
//    4 workgroups with no LDS). They perform the same fp32 operations in the same order,
//    so a request's results do not depend on which one runs: not on the
//    batch size, nor on how its tokens are split over calls.

#include <hip/hip_runtime.h>
#include <stdint.h>


#include "la_decode.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

enum Variant { VAR_LA = 0, VAR_GDN = 1, VAR_KDA = 2 };

// Tunables (compile-time; the defaults are the measured best on MI355X).
#ifndef LA_ROWS_PER_WAVE
#define LA_ROWS_PER_WAVE 32  // state rows a wave keeps in VGPRs: 8, 16 or 32
#endif
#ifndef LA_WAVES_PER_EU
#define LA_WAVES_PER_EU 0  // >0: ask the register allocator for this occupancy
#endif

constexpr int kRowsPerWave = LA_ROWS_PER_WAVE;
// Rows per wave of calls that write update records (speculative verify):
// twice the waves per tile and a smaller register footprint than 32 rows
// (occupancy 4 instead of 3 for KDA). Measured on MI355X, KDA B=64 T=4
// verify + replay: 63.3 -> 61.0 us per step (64.9 -> 67.3 % of peak); plain
// calls keep kRowsPerWave (KDA B=256 T=1: 32 rows 144.2 us, 16 rows 155.0).
constexpr int kRecordRowsPerWave = 16;
// Rows per wave of grids that fill less than one resident round: the same
// tiles over twice the waves keep more loads in flight on an underfilled
// chip. Used while B * HV * (V / 16) <= kSmallGridWaves, which at V = 128
// is 512 tiles: 4096 waves, the resident capacity of this instance (82-89
// VGPRs, two 8-wave workgroups per CU, 4 waves per SIMD), where 32 rows per
// wave leave at most 2 waves per SIMD. Measured on MI355X, % of peak HBM bandwidth,
// 32 -> 16 rows: GDN B=16 HV=32 63.5 -> 66.9; KDA B=16 H=24 62.4 -> 64.6;
// GDN B=64 HV=8 63.7 -> 66.2; GDN B=16 HV=32 T=4 53.6 -> 65.7; KDA B=16
// H=24 T=8 35.6 -> 43.8; GDN K=V=64 B=32 HV=32 T=4 42.0 -> 49.5. Two
// grids lost 1-3 % (Lightning B=33 H=8 47.2 -> 46.3; GDN B=32 HV=8 T=4
// with the cache 62.5 -> 60.9). At 768 tiles two rounds are needed and 16
// rows lose (GDN B=24 HV=32: 72.5 -> 62.7).
constexpr int kSmallGridRowsPerWave = 16;
constexpr int64_t kSmallGridWaves = 4096;
// Pairs per XCD block (xcd_block_pair): calls with fewer value heads than
// kXcdRangeMaxHeads give each XCD one contiguous range of pairs, i.e. whole
// requests; the others deal blocks of kXcdBlockPairs pairs (exceptions in
// select_kernel). See xcd_block_for for the measurements.
constexpr int kXcdRangeMaxHeads = 48;
constexpr int kXcdBlockPairs = 32;
// Workgroups per K = V = 128 tile of the one-token kernel: its waves are
// independent (no LDS, no barrier), so a tile's 16 waves run as
// 2^kOneSplitLog2 workgroups, and each XCD takes whole tiles in turn (the
// parts of a tile share an L2 for its q, k, v). Measured on MI355X at
// steady clocks, % of peak HBM bandwidth, one workgroup per tile (XCD
// ranges or 32-pair blocks) -> 4 workgroups in whole tiles: GDN B=64 HV=32
// 69.9 -> 74.6, Lightning B=33 H=64 74.9 -> 79.3 (2 workgroups in XCD
// ranges or blocks: 71.4 and 77.8; 8 workgroups: 70.8 and 73.6; 4
// workgroups in XCD ranges or blocks of tiles: 74.5 and 78.0, better only
// at 16 value heads). Other tile shapes keep one workgroup per tile in XCD
// ranges (K = V = 64, GDN B=256 HV=32, us per call: 46.2; split in 2 or 4
// workgroups: 51.9 and 52.6; K = 64, V = 128: 89.0 against 91.1 split in
// 4).
#ifndef LA_ONE_SPLIT_LOG2
#define LA_ONE_SPLIT_LOG2 2
#endif
constexpr int kOneSplitLog2 = LA_ONE_SPLIT_LOG2;
// Whole tiles per XCD block of the split one-token kernel. Same box, steady
// clocks, us per call, 1 tile per block -> 4: GDN B=64 HV=32 45.8 -> 45.5,
// Lightning B=33 H=64 44.3 -> 43.9, KDA B=256 H=24 137.3 -> 134.7, GDN
// B=256 HV=16 95.4 -> 93.5, GDN B=128 HV=32 88.4 -> 87.8, bf16 GDN B=128
// HV=32 46.6 -> 45.6. Two tiles fell between, eight matched four, 16 and 32
// lost at 32 heads (GDN B=64: 46.4, 47.0) and a whole request per block
// lost more (GDN B=64 46.9, Lightning 47.8).
constexpr int kOneXcdTiles = 4;
// Largest grid of the packed bf16 one-token kernel: what one resident round
// of it holds on 256 CUs (eight 2-wave workgroups per CU at 4 waves per SIMD;
// six for the KDA instance at 3). The one-token kernel takes larger grids.
constexpr int64_t kPackedMaxTiles = 2048;
constexpr int64_t kPackedMaxTilesKda = 1536;
static_assert(kRowsPerWave == 8 || kRowsPerWave == 16 || kRowsPerWave == 32,
              "8, 16 or 32 rows");
constexpr int kTokChunk = 8;
// Tokens per LDS round of 32-row grids that write a state per token (cache or
// paged slots). Why two tokens per round beat eight there is not
// established: an extra barrier every two tokens alone did not reproduce
// the gain, so it is the interleaving of the later tokens' prologue with
// the state writes rather than the synchronisation. Measured on MI355X,
// % of peak HBM bandwidth, 8 -> 2 tokens per round: GDN B=32 HV=32 T=4 with the cache 66.9 -> 70.6; paged GDN B=64
// T=4 67.2 -> 69.9; Lightning B=16 H=64 T=4 with the cache 68.5 -> 71.6;
// GDN B=32 T=8 with the cache 71.3 -> 73.0; KDA B=64 T=4 with the cache
// 67.4 -> 68.4. Varlen batches (T_b ~ U{1..4}) lost 0.4-0.6 points and keep
// eight; without per-token writes fewer tokens per round lose (update
// records: KDA B=64 T=4 verify + replay 67.9 -> 62.3).
constexpr int kCacheTokChunk = 2;
// Tokens per LDS round of 32-row KDA grids with more than four tokens and no
// per-token state writes. Measured on MI355X at steady clocks (HIP events
// over 200 calls, 5 rotating pool copies), KDA B=256 H=24 T=8, us per call
// in two runs: 8 tokens per round 171.4 and 170.8, 4 tokens 165.6 and 165.6,
// 2 tokens 171.5 and 171.5. 16 rows per wave with 8 tokens per round gained
// 0.3-1.2 % at T=8 (164.3) but lost 7-12 % at T=12 and 16, and the tile
// split over 2 or 4 workgroups (each forming every token's record) lost
// 7 and 18 %. GDN keeps 8 tokens per round (B=64 HV=32 T=8: 59.4 against
// 62.5 with 4; B=128: 109.5 against 113.2).
constexpr int kKdaTokChunk = 4;
constexpr float kL2Eps = 1e-6f;
// Final write-back of the general kernel's 32-row instances without
// per-token writes (fp32 K = V = 128 tiles): each wave passes its rows, 8 at
// a time, through its own LDS area and writes them with instructions that
// cover 2 whole rows (512 B each) instead of 8 128-byte row pieces. Rows
// are kStageRowFloats apart in the area (4 floats of padding). Same box,
// steady clocks, us per call, direct -> staged (two runs): KDA B=256 H=24
// T=8 165.2 -> 163.0, KDA B=128 T=8 90.0 -> 88.5, GDN B=64 HV=32 T=8 60.1 ->
// 58.3, T=2 48.6 -> 48.1, GDN B=32 HV=32 T=1 24.0 -> 23.0, Lightning B=15
// H=64 23.4 -> 23.0; the varlen GDN batch with the cache even (110.1 and
// 110.4). Not used where it did not gain: the 16-row instance (KDA B=16 T=8
// 15.5 -> 16.1) and the two-token instance that writes every token's state
// (GDN B=32 T=4 with the cache: final write-back staged 69.1 -> 69.6; every
// token's state staged as well 67.3 against 68.9 on one box, 69.1 against
// 68.8-69.3 on another, with 24 scalar registers spilled to vector lanes).
// Loading the tile the same way (contiguous loads, transposed through LDS
// before the token loop) lost everywhere (KDA T=8 170.1, GDN T=1 24.6). Instances with bf16 outputs
// keep direct stores: their token loop leaves no registers to spare, and
// the staging took three of them past 128 VGPRs (3 waves per SIMD).
constexpr int kStageRowFloats = 132;
template <int K, int V, bool BF16OUT, bool BF16S, bool REC, int R, int CH>
constexpr bool staged_writeback()
{
    return !BF16S && !BF16OUT && !REC && K == 128 && V == 128 && R == 32 &&
           CH != kCacheTokChunk;
}

// Activation strides are 32-bit: the host checks that every element offset
// of q, k, v, g, beta and out fits in 31 bits (the pool keeps 64-bit
// strides), which keeps the kernels' scalar registers within budget.
struct Params {
    int32_t B, T, HV, group;  // group = HV / H
    uint32_t flags;
    const void *q;
    int32_t sq_b, sq_t, sq_h;
    const void *k;
    int32_t sk_b, sk_t, sk_h;
    const void *v;
    int32_t sv_b, sv_t, sv_h;
    const float *g;
    int32_t sg_b, sg_t, sg_h;
    const float *beta;
    int32_t sb_b, sb_t, sb_h;
    void *pool;  // fp32 or bf16 elements (state dtype)
    int64_t sp_slot, sp_head, sp_row;
    const int32_t *ridx;
    const int32_t *widx;
    void *inter;  // state dtype
    void *out;
    int32_t so_b, so_t, so_h;
    const int32_t *tslots;  // paged per-token slot table, or null
    int64_t ts_stride;
    const int32_t *naccept;
    float *factors;  // [B, T, HV, 2K + V] per-token records, or null
    const int32_t *cu;  // [B + 1] token offsets of a varlen batch, or null
    int32_t total;      // rows of the token-packed arrays (with cu)
    int32_t gate;       // gate chain: 0 off, 1 softplus form, 2 bounded form
    const float *A_log;    // [HV]
    const float *dt_bias;  // [HV] (GDN) or [HV, K] (KDA)
    float lower_bound;
    int32_t xcd_block;  // pairs per block dealt to the XCDs (pair_of_block)
    int32_t split_log2;  // decode1_kernel: log2 of the workgroups per tile
};

// ---------------------------------------------------------------- helpers

// The dispatcher hands workgroup i to XCD i % 8 (eight XCDs, round robin).
// Workgroups take their (request, value head) pairs in blocks of C
// consecutive pairs dealt round robin to the XCDs: XCD x gets blocks x,
// x + 8, ... C = 1 is the plain order (each XCD takes every eighth pair);
// C = n / 8 gives each XCD one contiguous range. Workgroups beyond the last
// whole round of 8 C keep the plain order, so the map is a permutation of
// [0, n) for every n and C >= 1.
__device__ __forceinline__ int xcd_block_pair(int i, int n, int C)
{
    const int nfull = (n / (8 * C)) * (8 * C);
    if (i >= nfull)
        return i;
    const int x = i & 7, g = i >> 3;
    return ((g / C) * 8 + x) * C + (g % C);
}

__device__ __forceinline__ int pair_of_block(int xcd_block)
{
    return xcd_block > 1 ? xcd_block_pair(blockIdx.x, gridDim.x, xcd_block)
                         : static_cast<int>(blockIdx.x);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_act(const void *base, int64_t i)
{
    if constexpr (BF16)
        return bf16_to_f32(static_cast<const uint16_t *>(base)[i]);
    else
        return static_cast<const float *>(base)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_out(void *base, int64_t i, float x)
{
    if constexpr (BF16)
        static_cast<uint16_t *>(base)[i] = f32_to_bf16(x);
    else
        static_cast<float *>(base)[i] = x;
}

// DPP lane moves inside groups of 8 lanes (bound_ctrl on, all rows/banks).
__device__ __forceinline__ float dpp_xor1(float x)
{
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x)
{
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_half_mirror(float x)
{
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
}

// Sum over the 8 lanes (lane & ~7) .. (lane | 7). Each step adds a lane
// pair's values in both lanes, so all 8 lanes end with the same bits.
__device__ __forceinline__ float sum8(float x)
{
    x += dpp_xor1(x);
    x += dpp_xor2(x);
    x += dpp_half_mirror(x);
    return x;
}

// Lane moves for rows spread over LPR = 8 NJ consecutive lanes, where lane
// c + 8 j of a row holds its 16-byte chunk c + 8 j (decode1_kernel).
// chunk_pass(x, s): lanes with j = s receive the value of lane c + 8 (s - 1):
// xor 8 inside a 16-lane row (DPP row_ror:8) for s = 1 and 3, xor 24 inside
// a 32-lane half (ds_swizzle) for s = 2. Other lanes receive values they do
// not use. s is a compile-time constant after unrolling.
__device__ __forceinline__ float chunk_pass(float x, int s)
{
    if (s == 2)
        return __int_as_float(
            __builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x601F));
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Every lane c + 8 j of a row takes the value of lane c + 8 (NJ - 1).
template <int NJ>
__device__ __forceinline__ float from_last_chunk(float x)
{
    if constexpr (NJ == 1)
        return x;
    else if constexpr (NJ == 2)  // lanes c take lane c + 8 (row_ror:8)
        // one DPP move whose bank mask (lanes 0-7 of each 16-lane row)
        // leaves lanes 8-15 their own value: no select, so the compiler
        // cannot narrow the exec mask under the move (a DPP read from an
        // inactive lane yields 0)
        return __int_as_float(__builtin_amdgcn_update_dpp(
            __float_as_int(x), __float_as_int(x), 0x128, 0xF, 0x3, false));
    else  // lane (lane & 0x07) | 0x18 of each 32-lane half (ds_swizzle)
        return __int_as_float(
            __builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x307));
}

// Sum over the whole wave (token prologues).
__device__ __forceinline__ float wave_sum(float x)
{
    x = sum8(x);
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Buffer resources: the tile base lives in SGPRs (uniform per workgroup),
// each lane adds one 32-bit byte offset, row groups add a uniform offset.
// Accesses past `bytes` read zero / are dropped by the hardware.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef unsigned u4 __attribute__((ext_vector_type(4)));
constexpr int kBufDword3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format
// Cache-policy bits of the state tile's buffer accesses (gfx950: 2 = nt,
// 16 = sc1). Every tile load streams: a tile is used once per call, and on
// MI355X streaming loads measured as fast as or faster than cached loads for
// every workload once the Infinity Cache cannot keep tiles between calls.
constexpr int kStreamPolicy = 2;
// Tile stores: nontemporal with the sc1 bit (16 | 2). Measured on MI355X with
// a 4 GiB rotation against plain nontemporal stores: +0.4 to +1.7 points of
// peak HBM bandwidth on every workload (Lightning B=33 H=64 74.1 -> 74.9 %,
// KDA B=256 T=1 69.3 -> 70.6 %, paged GDN 63.6 -> 65.2 %), except the packed
// bf16 kernel (66.1 -> 64.8 %), which keeps kStreamPolicy. sc1 alone, or sc0
// with or without it and without nt, was 1-9 points slower.
constexpr int kStorePolicy = 18;
// Tile loads of a call that writes update records: ordinary cached loads.
// Such a call is a speculative verify, and the replay that follows re-reads
// the same seed tiles, which then come from the Infinity Cache. Measured on
// MI355X (verify + replay, 4 GiB rotation between steps, % of peak HBM
// bandwidth on the algorithmic bytes): KDA B=64 T=4 60.6 -> 64.9, KDA B=256
// 68.1 -> 72.4, GDN B=64 64.2 -> 68.6, KDA with a bf16 pool 48.5 -> 50.2.
constexpr int kRecordLoadPolicy = 0;

__device__ __forceinline__ BufRsrc make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base),
                                             static_cast<short>(0),
                                             static_cast<int>(bytes),
                                             kBufDword3);
}

// 128-bit store of the tile: `lane` = the lane's byte offset, `soff` = a
// uniform (row) offset. A store wider than 64 bits may read its data VGPRs
// after it issues, so a VALU write to them needs one wait state in between.
// The compiler inserts that wait only for buffer stores whose soffset is not
// an SGPR, so the whole offset goes in voffset and soffset stays the constant
// 0. The empty asm makes `soff` opaque at each store, so the VGPR sum is
// formed there and dies there instead of being hoisted and held in a VGPR.
template <int POLICY = kStorePolicy>
__device__ __forceinline__ void store_b128(u4 x, BufRsrc r, uint32_t lane,
                                           uint32_t soff)
{
    asm volatile("" : "+s"(soff));
    __builtin_amdgcn_raw_buffer_store_b128(x, r, lane + soff, 0, POLICY);
}

typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

// State tile I/O in the pool's element type. Every lane moves whole
// 16-byte chunks (128-bit buffer loads and stores): chunk j of lane c holds
// elements (c + 8 j) * 16/ES ... of a row, so a wave instruction covers eight
// full 128-byte row segments in either dtype. In registers a lane keeps its
// columns as groups of four fp32 values: one group per chunk for fp32, two
// for bf16 (widened exactly on load, rounded to nearest even on store by
// v_cvt_pk_bf16_f32). All arithmetic stays fp32.
template <bool BF16S>
struct StateIO {
    static constexpr uint32_t ES = BF16S ? 2u : 4u;  // bytes per element
    static constexpr int GPC = BF16S ? 2 : 1;         // 4-col groups / chunk

    // first column of the lane's 4-column group m
    static __device__ __forceinline__ int col(int m, int c8)
    {
        return (c8 + 8 * (m / GPC)) * (4 * GPC) + 4 * (m % GPC);
    }

    // one row: `lane` = the lane's byte offset in the row, `soff` = the
    // row's uniform offset; the groups of chunk j sit j * 128 bytes further
    template <int POLICY, int CPL>
    static __device__ __forceinline__ void load_row(f4 (&x)[CPL], BufRsrc r,
                                                    uint32_t lane,
                                                    uint32_t soff)
    {
#pragma unroll
        for (int j = 0; j < CPL / GPC; ++j) {
            const u4 h = __builtin_amdgcn_raw_buffer_load_b128(
                r, lane + j * 128u, soff, POLICY);
            if constexpr (BF16S) {
                x[2 * j] = f4{__uint_as_float(h.x << 16),
                              __uint_as_float(h.x & 0xffff0000u),
                              __uint_as_float(h.y << 16),
                              __uint_as_float(h.y & 0xffff0000u)};
                x[2 * j + 1] = f4{__uint_as_float(h.z << 16),
                                  __uint_as_float(h.z & 0xffff0000u),
                                  __uint_as_float(h.w << 16),
                                  __uint_as_float(h.w & 0xffff0000u)};
            } else {
                x[j] = __builtin_bit_cast(f4, h);
            }
        }
    }

    template <int CPL>
    static __device__ __forceinline__ void store_row(BufRsrc r, uint32_t lane,
                                                     uint32_t soff,
                                                     const f4 (&x)[CPL])
    {
#pragma unroll
        for (int j = 0; j < CPL / GPC; ++j) {
            u4 h;
            if constexpr (BF16S) {
                h.x = pack(x[2 * j].x, x[2 * j].y);
                h.y = pack(x[2 * j].z, x[2 * j].w);
                h.z = pack(x[2 * j + 1].x, x[2 * j + 1].y);
                h.w = pack(x[2 * j + 1].z, x[2 * j + 1].w);
            } else {
                h = __builtin_bit_cast(u4, x[j]);
            }
            store_b128(h, r, lane + j * 128u, soff);
        }
    }

    static __device__ __forceinline__ unsigned pack(float lo, float hi)
    {
        const f2 v = {lo, hi};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf2));
    }
};

// LDS-only barrier: orders LDS traffic across the workgroup without
// waiting for outstanding global loads (the state tile may still be in
// flight while the prologue runs).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Order one wave's LDS accesses to an area only it uses: what its lanes
// wrote before is visible to all its lanes after (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// LDS record of one token: k^[K], q^[K], (KDA: e[K]), v[V] (rows permuted so
// each lane's rows are adjacent), and 4 scalars (beta, decay, k^.q^, pad).
template <int VAR, int K, int V>
struct TokLayout {
    static constexpr int kOff = 0;
    static constexpr int qOff = K;
    static constexpr int eOff = 2 * K;
    static constexpr int vOff = (VAR == VAR_KDA ? 3 : 2) * K;
    static constexpr int sOff = vOff + V;
    static constexpr int size = sOff + 4;  // floats; a multiple of 4
};

// Position of state row `row` inside the LDS v record: the rows a lane owns
// (R w + 8 i + r, i = 0..R/8-1, R rows per wave) sit at R w + (R/8) r + i.
template <int R>
__device__ __forceinline__ int v_slot(int row)
{
    constexpr int RPL = R / 8;
    const int w = row / R, i = (row % R) / 8, r = row % 8;
    return w * R + r * RPL + i;
}

// Raw per-token inputs one lane loads for the prologue.
template <int K, int V>
struct TokRaw {
    float q[K / 64], k[K / 64], e[K / 64], v[V / 64];
    float g, beta;
};

// Log-decay of the gate chain for z = raw gate + dt_bias:
// -exp(A_log) softplus(z), or lower_bound sigmoid(exp(A_log) z) in the
// bounded form. Hardware exp, log and reciprocal (about 1 ulp each):
// softplus(z) = log(1 + e^z) loses only terms below 2^-24 of the decay, and
// z > 20 takes softplus = z.
__device__ __forceinline__ float gate_chain(const Params &p, float z,
                                            float a_log)
{
    const float a = __expf(a_log);
    if (p.gate == 2)
        return p.lower_bound *
               __builtin_amdgcn_rcpf(1.f + __expf(-a * z));
    const float sp = z > 20.f ? z : __logf(1.f + __expf(z));
    return -a * sp;
}

// First half of the prologue of token t: global loads only, so they can be
// issued ahead of the state tile and arrive first.
template <int VAR, int K, int V, bool BF16IN>
__device__ __forceinline__ void prologue_load(const Params &p, int b, int hv,
                                              int t, int lane,
                                              TokRaw<K, V> &raw)
{
    constexpr int EPL = K / 64;  // key elements per lane
    constexpr int VPL = V / 64;  // value elements per lane
    const int h = hv / p.group;
    const int32_t qo = b * p.sq_b + t * p.sq_t + h * p.sq_h;
    const int32_t ko = b * p.sk_b + t * p.sk_t + h * p.sk_h;
    const int32_t vo = b * p.sv_b + t * p.sv_t + hv * p.sv_h;
    const int32_t go = b * p.sg_b + t * p.sg_t + hv * p.sg_h;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        raw.q[i] = load_act<BF16IN>(p.q, qo + lane * EPL + i);
        raw.k[i] = load_act<BF16IN>(p.k, ko + lane * EPL + i);
        if constexpr (VAR == VAR_KDA) {
            // with the gate chain: z = raw gate + dt_bias of the channel
            raw.e[i] = p.g[go + lane * EPL + i] +
                       (p.gate ? p.dt_bias[hv * K + lane * EPL + i] : 0.f);
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        raw.v[i] = load_act<BF16IN>(p.v, vo + lane * VPL + i);
    if constexpr (VAR == VAR_LA) {
        raw.g = p.g ? p.g[hv] : 0.f;
        raw.beta = 1.f;
    } else {
        raw.g = (VAR == VAR_GDN)
                    ? p.g[go] + (p.gate ? p.dt_bias[hv] : 0.f)
                    : 0.f;
        raw.beta = p.beta[b * p.sb_b + t * p.sb_t + hv * p.sb_h];
    }
}

// Second half: l2norm, k.q, sigmoid, exp; writes the LDS record `rec` (v
// rows placed for R rows per wave) and, when `frec` is set, the decay and
// key of the token's update record.
template <int VAR, int K, int V, int R = kRowsPerWave>
__device__ __forceinline__ void prologue_finish(const Params &p, int hv,
                                                int lane,
                                                const TokRaw<K, V> &raw,
                                                float *rec, float *frec)
{
    using L = TokLayout<VAR, K, V>;
    constexpr int EPL = K / 64;
    constexpr int VPL = V / 64;
    float ssq = 0.f, ssk = 0.f, qk = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        ssq = fmaf(raw.q[i], raw.q[i], ssq);
        ssk = fmaf(raw.k[i], raw.k[i], ssk);
        qk = fmaf(raw.q[i], raw.k[i], qk);
    }
    float rq = 1.f, rk = 1.f;
    qk = wave_sum(qk);
    if (p.flags & LA_F_L2NORM_QK) {
        ssq = wave_sum(ssq);
        ssk = wave_sum(ssk);
        rq = __frsqrt_rn(ssq + kL2Eps);
        rk = __frsqrt_rn(ssk + kL2Eps);
    }
    // the scalar decay (GDN, Lightning), identical in every lane
    float decay;
    if constexpr (VAR == VAR_LA)
        decay = p.g ? raw.g
                    : __expf(-exp2f(-8.f * static_cast<float>(hv + 1) /
                                    static_cast<float>(p.HV)));
    else if constexpr (VAR == VAR_GDN)
        decay = __expf(p.gate ? gate_chain(p, raw.g, p.A_log[hv]) : raw.g);
    else
        decay = 1.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int j = lane * EPL + i;
        const float kn = raw.k[i] * rk;
        rec[L::kOff + j] = kn;
        rec[L::qOff + j] = raw.q[i] * rq;
        float a = decay;
        if constexpr (VAR == VAR_KDA) {
            a = __expf(p.gate ? gate_chain(p, raw.e[i], p.A_log[hv])
                              : raw.e[i]);
            rec[L::eOff + j] = a;
        }
        if (frec) {
            frec[j] = a;
            frec[K + j] = kn;
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        rec[L::vOff + v_slot<R>(lane * VPL + i)] = raw.v[i];
    if (lane == 0) {
        float beta = 1.f;
        if constexpr (VAR != VAR_LA)
            beta = (p.flags & LA_F_BETA_LOGIT)
                       ? 1.f / (1.f + __expf(-raw.beta))
                       : raw.beta;
        rec[L::sOff + 0] = beta;
        rec[L::sOff + 1] = decay;
        rec[L::sOff + 2] = qk * rq * rk;
        rec[L::sOff + 3] = 0.f;
    }
}

// Start of the update record of flat token `tok` (b T + t, or the packed
// token number of a varlen batch) and value head hv.
template <int K, int V>
__device__ __forceinline__ float *factor_record(const Params &p, int64_t tok,
                                                int hv)
{
    return p.factors +
           (tok * p.HV + hv) * static_cast<int64_t>(2 * K + V);
}

// Token range of request b: its count, the offset added to t in the
// per-token arrays and the flat number of its token 0 (b T in a dense batch).
// False when varlen offsets break the precondition (the request is skipped).
__device__ __forceinline__ bool request_tokens(const int32_t *cu, int32_t total,
                                               int b, int T, int &Tb,
                                               int &tok0, int64_t &flat0)
{
    Tb = T;
    tok0 = 0;
    flat0 = static_cast<int64_t>(b) * T;
    if (!cu)
        return true;
    const int c0 = __builtin_amdgcn_readfirstlane(cu[b]);
    const int c1 = __builtin_amdgcn_readfirstlane(cu[b + 1]);
    if (c0 < 0 || c1 < c0 || c1 > total || c1 - c0 > T)
        return false;
    Tb = c1 - c0;
    tok0 = c0;
    flat0 = c0;
    return true;
}

#if LA_WAVES_PER_EU > 0
#define LA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(LA_WAVES_PER_EU)))
#else
#define LA_OCCUPANCY
#endif

// REC: also write the per-token update records (a separate instantiation so
// that the ordinary path carries none of their register cost). R: state rows
// per wave (the workgroup has V / R waves); it only distributes rows over
// waves, each row's arithmetic is the same for every R.
template <int VAR, int K, int V, bool BF16IN, bool BF16OUT, bool BF16S,
          bool REC, int R, int CH>
__global__ void __launch_bounds__((V / R) * 64) LA_OCCUPANCY
decode_kernel(const Params p)
{
    using IO = StateIO<BF16S>;
    constexpr uint32_t ES = IO::ES;
    extern __shared__ f4 lds_raw[];
    float *lds = reinterpret_cast<float *>(lds_raw);
    using L = TokLayout<VAR, K, V>;
    constexpr int NW = V / R;  // waves per workgroup
    constexpr int RPL = R / 8;  // rows per lane
    constexpr int CPL = K / 32;            // 16-byte chunks per lane and row

    const int pair = pair_of_block(p.xcd_block);
    const int b = pair / p.HV;
    const int hv = pair - b * p.HV;
    const int lane = threadIdx.x & 63;
    // wave index and slots are uniform across the wave; saying so keeps the
    // buffer descriptors and row offsets in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c8 = lane & 7;
    const int rs = lane >> 3;
    const int T = p.T;
    int Tb, tok0;
    int64_t flat0;
    if (!request_tokens(p.cu, p.total, b, T, Tb, tok0, flat0))
        return;

    int r, w;
    if (p.tslots) {
        // paged slots: seed = entry of the last accepted token; the state is
        // written after every token instead of once at the end
        const int na = __builtin_amdgcn_readfirstlane(p.naccept[b]);
        r = (na >= 1 && na <= Tb)
                ? __builtin_amdgcn_readfirstlane(p.tslots[b * p.ts_stride + na - 1])
                : -1;
        w = -1;
    } else {
        r = __builtin_amdgcn_readfirstlane(p.ridx[b]);
        w = __builtin_amdgcn_readfirstlane(p.widx ? p.widx[b] : r);
    }

    // Output row written by this lane (lanes with c8 < RPL cover the wave's
    // rows exactly once): row R wave + 8 c8 + rs.
    const int orow = wave * R + (c8 & (RPL - 1)) * 8 + rs;
    const bool olane = c8 < RPL;
    const int32_t obase = b * p.so_b + tok0 * p.so_t + hv * p.so_h + orow;

    if (r < 0) {  // padded request: zero outputs, touch nothing else
        if (olane)
            for (int t = 0; t < Tb; ++t)
                store_out<BF16OUT>(p.out, obase + t * p.so_t, 0.f);
        return;
    }

    // Gather the tile rows this lane owns: 128-bit buffer loads from the
    // read tile; the lane's part of the address is one 32-bit offset. They
    // are requested before the token inputs: the tile is the bulk of the
    // call's traffic (requesting the inputs ahead of it measured slower).
    const uint32_t row_bytes = static_cast<uint32_t>(p.sp_row) * ES;
    const uint32_t tile_bytes = static_cast<uint32_t>(
        (static_cast<int64_t>(V - 1) * p.sp_row + K) * ES);
    const uint32_t lane_off = rs * row_bytes + c8 * 16u;
    char *const pool = static_cast<char *>(p.pool);
    const BufRsrc src = make_rsrc(
        pool + (r * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
    f4 S[RPL][CPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        IO::template load_row<REC ? kRecordLoadPolicy : kStreamPolicy>(
            S[i], src, lane_off, (wave * R + i * 8) * row_bytes);

    for (int t0 = 0; t0 < Tb; t0 += CH) {
        const int nt = min(CH, Tb - t0);
        if (t0 > 0)
            lds_barrier();  // every wave is done with the previous chunk
        for (int tt = wave; tt < nt; tt += NW) {
            TokRaw<K, V> rw;
            prologue_load<VAR, K, V, BF16IN>(p, b, hv, tok0 + t0 + tt, lane,
                                             rw);
            prologue_finish<VAR, K, V, R>(
                p, hv, lane, rw, lds + tt * L::size,
                REC ? factor_record<K, V>(p, flat0 + t0 + tt, hv) : nullptr);
        }
        lds_barrier();

        for (int tt = 0; tt < nt; ++tt) {
            const int t = t0 + tt;
            const float *rec = lds + tt * L::size;
            const float beta = rec[L::sOff + 0];
            const float decay = rec[L::sOff + 1];
            const float kq = rec[L::sOff + 2];
            float vr[RPL];
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                vr[i] = rec[L::vOff + wave * R + rs * RPL + i];

            // decay
            if constexpr (VAR == VAR_KDA) {
#pragma unroll
                for (int m = 0; m < CPL; ++m) {
                    const f4 e = *reinterpret_cast<const f4 *>(
                        rec + L::eOff + IO::col(m, c8));
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
                        S[i][m] *= e;
                }
            } else {
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int m = 0; m < CPL; ++m)
                        S[i][m] *= decay;
            }

            // read-outs u = S k (delta rules) and w = S q
            f4 kk[CPL];
            float u[RPL], wq[RPL];
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                u[i] = 0.f;
                wq[i] = 0.f;
            }
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                kk[m] = *reinterpret_cast<const f4 *>(
                    rec + L::kOff + IO::col(m, c8));
                const f4 qq = *reinterpret_cast<const f4 *>(
                    rec + L::qOff + IO::col(m, c8));
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    if constexpr (VAR != VAR_LA) {
                        u[i] = fmaf(S[i][m].x, kk[m].x, u[i]);
                        u[i] = fmaf(S[i][m].y, kk[m].y, u[i]);
                        u[i] = fmaf(S[i][m].z, kk[m].z, u[i]);
                        u[i] = fmaf(S[i][m].w, kk[m].w, u[i]);
                    }
                    wq[i] = fmaf(S[i][m].x, qq.x, wq[i]);
                    wq[i] = fmaf(S[i][m].y, qq.y, wq[i]);
                    wq[i] = fmaf(S[i][m].z, qq.z, wq[i]);
                    wq[i] = fmaf(S[i][m].w, qq.w, wq[i]);
                }
            }
            float c[RPL], o[RPL];
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                wq[i] = sum8(wq[i]);
                if constexpr (VAR == VAR_LA) {
                    c[i] = vr[i];
                } else {
                    u[i] = sum8(u[i]);
                    c[i] = beta * (vr[i] - u[i]);
                }
                o[i] = fmaf(c[i], kq, wq[i]);
            }

            // rank-1 update S += c k^T
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int m = 0; m < CPL; ++m) {
                    S[i][m].x = fmaf(c[i], kk[m].x, S[i][m].x);
                    S[i][m].y = fmaf(c[i], kk[m].y, S[i][m].y);
                    S[i][m].z = fmaf(c[i], kk[m].z, S[i][m].z);
                    S[i][m].w = fmaf(c[i], kk[m].w, S[i][m].w);
                }

            // output: lane (c8, rs) with c8 < RPL writes row R w + 8 c8 + rs
            float mine = o[0];
#pragma unroll
            for (int i = 1; i < RPL; ++i)
                mine = (c8 == i) ? o[i] : mine;
            if (olane)
                store_out<BF16OUT>(p.out, obase + t * p.so_t, mine);
            if constexpr (REC) {
                // err of row orow, by the lane that writes its output
                float cm = c[0];
#pragma unroll
                for (int i = 1; i < RPL; ++i)
                    cm = (c8 == i) ? c[i] : cm;
                if (olane)
                    factor_record<K, V>(p, flat0 + t, hv)[2 * K + orow] = cm;
            }

            if (p.tslots) {
                const int ws = __builtin_amdgcn_readfirstlane(
                    p.tslots[b * p.ts_stride + t]);
                if (ws >= 0) {
                    const BufRsrc dst = make_rsrc(
                        pool + (ws * p.sp_slot + hv * p.sp_head) * ES,
                        tile_bytes);
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
                        IO::store_row(dst, lane_off,
                                      (wave * R + i * 8) * row_bytes,
                                      S[i]);
                }
            }

            if (p.inter) {
                // contiguous [B, T, HV, V, K] cache: rows are K floats apart
                const BufRsrc dst = make_rsrc(
                    static_cast<char *>(p.inter) +
                        ((flat0 + t) * p.HV + hv) *
                            static_cast<int64_t>(V * K * ES),
                    V * K * ES);
                const uint32_t ioff = rs * (K * ES) + c8 * 16u;
#pragma unroll
                for (int i = 0; i < RPL; ++i)
                    IO::store_row(dst, ioff,
                                  (wave * R + i * 8) * K * ES, S[i]);
            }
        }
    }

    if (w >= 0) {  // in-place writeback to the write slot
        const BufRsrc dst = make_rsrc(
            pool + (w * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
        if constexpr (staged_writeback<K, V, BF16OUT, BF16S, REC, R, CH>()) {
            // this wave's area follows the token records; lane l stores
            // 16-byte chunk l % 32 of row l / 32 of each row pair
            float *stage = lds + (T < CH ? T : CH) * L::size +
                           wave * (8 * kStageRowFloats);
            const int pr = lane >> 5, pc = lane & 31;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
#pragma unroll
                for (int m = 0; m < CPL; ++m)
                    *reinterpret_cast<f4 *>(stage + rs * kStageRowFloats +
                                            (c8 + 8 * m) * 4) = S[i][m];
                wave_lds_sync();  // the wave's writes before its reads
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    store_b128(__builtin_bit_cast(
                                   u4, *reinterpret_cast<const f4 *>(
                                           stage +
                                           (2 * j + pr) * kStageRowFloats +
                                           pc * 4)),
                               dst, pr * row_bytes + pc * 16u,
                               (wave * R + i * 8 + 2 * j) * row_bytes);
                wave_lds_sync();  // its reads before the next rows' writes
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                IO::store_row(dst, lane_off,
                              (wave * R + i * 8) * row_bytes, S[i]);
        }
    }
}

// One token on a bf16 pool, with no per-token state writes: the tile stays
// packed in registers (two bf16 per VGPR) and each element is widened where
// it is used, so a wave holds 64 rows in the registers that 32 fp32 rows
// take in decode_kernel, and twice as many tile bytes are in flight per
// compute unit. The arithmetic and its order are those of decode_kernel for
// T = 1 (widen, decay, dot products, rank-1 FMA, one rounding on store), so
// the two kernels give identical bits.
template <int VAR, int K, int V, bool BF16IN, bool BF16OUT>
__global__ void __launch_bounds__(V) decode_packed_kernel(const Params p)
{
    constexpr int R = 64;        // rows per wave
    constexpr int RPL = R / 8;   // rows per lane
    constexpr int NCH = K / 64;  // 16-byte chunks (8 columns) per lane and row
    constexpr uint32_t ES = 2;
    using L = TokLayout<VAR, K, V>;
    extern __shared__ f4 lds_raw[];
    float *lds = reinterpret_cast<float *>(lds_raw);

    const int pair = pair_of_block(p.xcd_block);
    const int b = pair / p.HV;
    const int hv = pair - b * p.HV;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c8 = lane & 7;
    const int rs = lane >> 3;

    const int r = __builtin_amdgcn_readfirstlane(p.ridx[b]);
    const int w = __builtin_amdgcn_readfirstlane(p.widx ? p.widx[b] : r);
    // every lane writes one output row: R wave + 8 c8 + rs
    const int32_t oidx = b * p.so_b + hv * p.so_h + wave * R + c8 * 8 + rs;
    if (r < 0) {
        store_out<BF16OUT>(p.out, oidx, 0.f);
        return;
    }

    // lane (c8, rs) holds rows R wave + 8 i + rs and the 16-byte chunks
    // c8 + 8 j of each: columns (c8 + 8 j) * 8 ... + 7
    const uint32_t row_bytes = static_cast<uint32_t>(p.sp_row) * ES;
    const uint32_t tile_bytes = static_cast<uint32_t>(
        (static_cast<int64_t>(V - 1) * p.sp_row + K) * ES);
    const uint32_t lane_off = rs * row_bytes + c8 * 16u;
    char *const pool = static_cast<char *>(p.pool);
    const BufRsrc src = make_rsrc(
        pool + (r * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
    u4 P[RPL][NCH];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < NCH; ++j)
            P[i][j] = __builtin_amdgcn_raw_buffer_load_b128(
                src, lane_off + j * 128u, (wave * R + i * 8) * row_bytes,
                kStreamPolicy);

    if (wave == 0) {
        TokRaw<K, V> rw;
        prologue_load<VAR, K, V, BF16IN>(p, b, hv, 0, lane, rw);
        prologue_finish<VAR, K, V, R>(p, hv, lane, rw, lds, nullptr);
    }
    lds_barrier();

    const float beta = lds[L::sOff + 0];
    const float decay = lds[L::sOff + 1];
    const float kq = lds[L::sOff + 2];
    auto colof = [&](int m) { return (c8 + 8 * (m / 2)) * 8 + 4 * (m % 2); };
    f4 kk[2 * NCH], qq[2 * NCH], ee[2 * NCH];
#pragma unroll
    for (int m = 0; m < 2 * NCH; ++m) {
        kk[m] = *reinterpret_cast<const f4 *>(lds + L::kOff + colof(m));
        qq[m] = *reinterpret_cast<const f4 *>(lds + L::qOff + colof(m));
        if constexpr (VAR == VAR_KDA)
            ee[m] = *reinterpret_cast<const f4 *>(lds + L::eOff + colof(m));
    }
    float vr[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        vr[i] = lds[L::vOff + wave * R + rs * RPL + i];

    // column group m of a row (half m % 2 of chunk m / 2), widened, decayed
    auto widen = [&](const u4 &x, int m) -> f4 {
        const unsigned a = (m % 2) ? x.z : x.x, c = (m % 2) ? x.w : x.y;
        f4 s = {__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u),
                __uint_as_float(c << 16), __uint_as_float(c & 0xffff0000u)};
        if constexpr (VAR == VAR_KDA)
            s *= ee[m];
        else
            s *= decay;
        return s;
    };

    const BufRsrc dst = make_rsrc(
        pool + ((w < 0 ? 0 : w) * p.sp_slot + hv * p.sp_head) * ES,
        tile_bytes);
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        float u = 0.f, wq = 0.f;
#pragma unroll
        for (int m = 0; m < 2 * NCH; ++m) {
            const f4 s = widen(P[i][m / 2], m);
            if constexpr (VAR != VAR_LA) {
                u = fmaf(s.x, kk[m].x, u);
                u = fmaf(s.y, kk[m].y, u);
                u = fmaf(s.z, kk[m].z, u);
                u = fmaf(s.w, kk[m].w, u);
            }
            wq = fmaf(s.x, qq[m].x, wq);
            wq = fmaf(s.y, qq[m].y, wq);
            wq = fmaf(s.z, qq[m].z, wq);
            wq = fmaf(s.w, qq[m].w, wq);
        }
        wq = sum8(wq);
        float c;
        if constexpr (VAR == VAR_LA) {
            c = vr[i];
        } else {
            u = sum8(u);
            c = beta * (vr[i] - u);
        }
        mine = (c8 == i) ? fmaf(c, kq, wq) : mine;

        if (w >= 0) {  // S <- decayed S + c k^T, rounded once, row i stored
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                f4 lo = widen(P[i][j], 2 * j), hi = widen(P[i][j], 2 * j + 1);
                lo.x = fmaf(c, kk[2 * j].x, lo.x);
                lo.y = fmaf(c, kk[2 * j].y, lo.y);
                lo.z = fmaf(c, kk[2 * j].z, lo.z);
                lo.w = fmaf(c, kk[2 * j].w, lo.w);
                hi.x = fmaf(c, kk[2 * j + 1].x, hi.x);
                hi.y = fmaf(c, kk[2 * j + 1].y, hi.y);
                hi.z = fmaf(c, kk[2 * j + 1].z, hi.z);
                hi.w = fmaf(c, kk[2 * j + 1].w, hi.w);
                u4 h;
                h.x = StateIO<true>::pack(lo.x, lo.y);
                h.y = StateIO<true>::pack(lo.z, lo.w);
                h.z = StateIO<true>::pack(hi.x, hi.y);
                h.w = StateIO<true>::pack(hi.z, hi.w);
                store_b128<kStreamPolicy>(h, dst, lane_off + j * 128u,
                                          (wave * R + i * 8) * row_bytes);
            }
        }
    }
    store_out<BF16OUT>(p.out, oidx, mine);
}

// One token with no per-token writes (any variant). Each load
// instruction of a wave reads 1 KiB of contiguous tile bytes (64 lanes x
// 16 B: 2 to 8 whole rows); on MI355X an in-place tile update moved that way
// keeps HBM busier than rows split into 128-byte pieces. A wave owns 8 rows,
// so a tile has V / 8 waves, run as 2^split_log2 workgroups (the waves share
// nothing). Lane (cl = lane % LPR, rl = lane / LPR)
// holds the 16-byte chunk cl of rows 8 wave + RPI j + rl (4 fp32 or 8 bf16
// columns, widened to fp32 in registers). Every wave forms the token
// prologue it needs itself (q and k, its rows of v, the scalars): no LDS and
// no barrier, and those loads are issued before the tile's. A bf16 state is
// rounded once, to nearest even, on store.
// The arithmetic repeats decode_kernel's at T = 1 operation for operation,
// in the same order, so a request gets the same bits from either kernel
// whatever the batch size or the split of its tokens over calls: the norms
// and k.q are summed over the wave with K / 64 elements per lane, as in the
// prologue, and a row's dot products run one FMA chain per c = cl & 7 over
// the chunks c, c + 8, ... (handed from lane to lane), closed by the same
// 8-lane butterfly. The extra lane moves cost ALU time that this
// memory-bound kernel has to spare.
template <int VAR, int K, int V, bool BF16IN, bool BF16OUT, bool BF16S>
__global__ void __launch_bounds__((V / 8) * 64) decode1_kernel(const Params p)
{
    constexpr uint32_t ES = BF16S ? 2u : 4u;  // state bytes per element
    constexpr int CPL = 16 / ES;    // columns per lane (one chunk per row)
    constexpr int G = CPL / 4;      // 4-column groups per chunk
    constexpr int LPR = K / CPL;    // lanes per row
    constexpr int RPI = 64 / LPR;   // rows per load instruction
    constexpr int RPL = 8 / RPI;    // rows per lane

    // workgroup -> (pair, part); part p of a tile split over 2^split_log2
    // workgroups takes the tile's waves p V / (8 2^split_log2) onwards
    const int blk = pair_of_block(p.xcd_block);
    const int pair = blk >> p.split_log2;
    const int part = blk - (pair << p.split_log2);
    const int b = pair / p.HV;
    const int hv = pair - b * p.HV;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(
        (threadIdx.x >> 6) + (part * (V / 8) >> p.split_log2));
    const int cl = lane % LPR;
    const int rl = lane / LPR;
    constexpr int NJ = LPR / 8;  // chunks c + 8 j per row and c
    const int c8 = cl & 7;
    const int jm = cl >> 3;

    const int r = __builtin_amdgcn_readfirstlane(p.ridx[b]);
    const int w = __builtin_amdgcn_readfirstlane(p.widx ? p.widx[b] : r);
    // lane c8 = j of a row's last chunk group writes the output of row j
    const bool olane = jm == NJ - 1 && c8 < RPL;
    const int orow = 8 * wave + RPI * (olane ? c8 : 0) + rl;
    const int32_t oidx = b * p.so_b + hv * p.so_h + orow;
    if (r < 0) {
        if (olane)
            store_out<BF16OUT>(p.out, oidx, 0.f);
        return;
    }

    // token inputs of this lane: q, k in the prologue's layout (K / 64
    // elements per lane, for the sums over K) and in the chunk layout
    constexpr int EPL = K / 64;
    const int h = hv / p.group;
    const int32_t qb = b * p.sq_b + h * p.sq_h;
    const int32_t kb = b * p.sk_b + h * p.sk_h;
    const int32_t vo = b * p.sv_b + hv * p.sv_h + 8 * wave + rl;
    const int32_t go = b * p.sg_b + hv * p.sg_h;
    float qe[EPL], ke[EPL], qv[CPL], kv[CPL], vv[RPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        qe[i] = load_act<BF16IN>(p.q, qb + lane * EPL + i);
        ke[i] = load_act<BF16IN>(p.k, kb + lane * EPL + i);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        qv[i] = load_act<BF16IN>(p.q, qb + CPL * cl + i);
        kv[i] = load_act<BF16IN>(p.k, kb + CPL * cl + i);
    }
#pragma unroll
    for (int j = 0; j < RPL; ++j)
        vv[j] = load_act<BF16IN>(p.v, vo + RPI * j);
    float gs = 0.f, bs = 1.f;
    if constexpr (VAR == VAR_GDN)
        gs = p.g[go] + (p.gate ? p.dt_bias[hv] : 0.f);
    if constexpr (VAR != VAR_LA)
        bs = p.beta[b * p.sb_b + hv * p.sb_h];
    // KDA: the raw gates (with dt_bias in the gate chain) in the
    // prologue's layout, K / 64 channels per lane, as prologue_load forms
    // them; read in the chunk layout instead, every lane would fetch 4 or 8
    // gates for 2 to 4 rows, as many load instructions as the tile takes
    float ev[EPL];
    if constexpr (VAR == VAR_KDA) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            ev[i] = p.g[go + lane * EPL + i] +
                    (p.gate ? p.dt_bias[hv * K + lane * EPL + i] : 0.f);
    }

    // the tile rows of this lane
    const uint32_t row_bytes = static_cast<uint32_t>(p.sp_row) * ES;
    const uint32_t tile_bytes = static_cast<uint32_t>(
        (static_cast<int64_t>(V - 1) * p.sp_row + K) * ES);
    const uint32_t lane_off = rl * row_bytes + cl * 16u;
    char *const pool = static_cast<char *>(p.pool);
    const BufRsrc src = make_rsrc(
        pool + (r * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
    f4 S[RPL][G];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const u4 x = __builtin_amdgcn_raw_buffer_load_b128(
            src, lane_off, (8 * wave + RPI * j) * row_bytes, kStreamPolicy);
        if constexpr (BF16S) {
            S[j][0] = f4{__uint_as_float(x.x << 16),
                         __uint_as_float(x.x & 0xffff0000u),
                         __uint_as_float(x.y << 16),
                         __uint_as_float(x.y & 0xffff0000u)};
            S[j][1] = f4{__uint_as_float(x.z << 16),
                         __uint_as_float(x.z & 0xffff0000u),
                         __uint_as_float(x.w << 16),
                         __uint_as_float(x.w & 0xffff0000u)};
        } else {
            S[j][0] = __builtin_bit_cast(f4, x);
        }
    }

    // prologue: l2norm over K, k.q, beta, decay
    float ssq = 0.f, ssk = 0.f, qk = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        ssq = fmaf(qe[i], qe[i], ssq);
        ssk = fmaf(ke[i], ke[i], ssk);
        qk = fmaf(qe[i], ke[i], qk);
    }
    float rq = 1.f, rk = 1.f;
    qk = wave_sum(qk);
    if (p.flags & LA_F_L2NORM_QK) {
        ssq = wave_sum(ssq);
        ssk = wave_sum(ssk);
        rq = __frsqrt_rn(ssq + kL2Eps);
        rk = __frsqrt_rn(ssk + kL2Eps);
    }
    const float kq = qk * rq * rk;
    f4 kk[G], qq[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        kk[g] = f4{kv[4 * g] * rk, kv[4 * g + 1] * rk, kv[4 * g + 2] * rk,
                   kv[4 * g + 3] * rk};
        qq[g] = f4{qv[4 * g] * rq, qv[4 * g + 1] * rq, qv[4 * g + 2] * rq,
                   qv[4 * g + 3] * rq};
    }
    // decay of each 4-column group: one factor (Lightning, GDN) or the
    // per-column KDA factors, computed as prologue_finish computes them
    f4 dec[G];
    if constexpr (VAR == VAR_KDA) {
        const float a_log = p.gate ? p.A_log[hv] : 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            ev[i] = __expf(p.gate ? gate_chain(p, ev[i], a_log) : ev[i]);
        // channel CPL cl + i of the chunk layout is element i % EPL of
        // lane (CPL cl + i) / EPL
        float e[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            e[i] = __shfl(ev[i % EPL], (CPL / EPL) * cl + i / EPL);
#pragma unroll
        for (int g = 0; g < G; ++g)
            dec[g] = f4{e[4 * g], e[4 * g + 1], e[4 * g + 2], e[4 * g + 3]};
    } else {
        float decay;
        if constexpr (VAR == VAR_LA)
            decay = p.g ? p.g[hv]
                        : __expf(-exp2f(-8.f * static_cast<float>(hv + 1) /
                                        static_cast<float>(p.HV)));
        else
            decay = __expf(p.gate ? gate_chain(p, gs, p.A_log[hv]) : gs);
#pragma unroll
        for (int g = 0; g < G; ++g)
            dec[g] = f4{decay, decay, decay, decay};
    }
    float beta = 1.f;
    if constexpr (VAR != VAR_LA)
        beta = (p.flags & LA_F_BETA_LOGIT) ? 1.f / (1.f + __expf(-bs)) : bs;

    // one FMA chain per row and c8 over chunks c8, c8 + 8, ...: in step s
    // the lanes of chunk c8 + 8 s extend the chain handed to them
    auto chain = [&](float acc, const f4 &x, const f4 &y) -> float {
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
        return acc;
    };
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
#pragma unroll
        for (int g = 0; g < G; ++g)
            S[j][g] *= dec[g];
        float u = 0.f, wq = 0.f;
#pragma unroll
        for (int st = 0; st < NJ; ++st) {
            if (st > 0) {
                if constexpr (VAR != VAR_LA)
                    u = chunk_pass(u, st);
                wq = chunk_pass(wq, st);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if constexpr (VAR != VAR_LA)
                    u = chain(u, S[j][g], kk[g]);
                wq = chain(wq, S[j][g], qq[g]);
            }
        }
        // the lanes of the last chunk group hold the chains; sum over c8
        wq = sum8(wq);
        float c;
        if constexpr (VAR == VAR_LA) {
            c = vv[j];
        } else {
            u = sum8(u);
            c = beta * (vv[j] - u);
        }
        mine = (jm == NJ - 1 && c8 == j) ? fmaf(c, kq, wq) : mine;
        if constexpr (VAR != VAR_LA)
            c = from_last_chunk<NJ>(c);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            S[j][g].x = fmaf(c, kk[g].x, S[j][g].x);
            S[j][g].y = fmaf(c, kk[g].y, S[j][g].y);
            S[j][g].z = fmaf(c, kk[g].z, S[j][g].z);
            S[j][g].w = fmaf(c, kk[g].w, S[j][g].w);
        }
    }
    if (olane)
        store_out<BF16OUT>(p.out, oidx, mine);
    if (w >= 0) {
        const BufRsrc dst = make_rsrc(
            pool + (w * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            u4 x;
            if constexpr (BF16S) {
                x.x = StateIO<true>::pack(S[j][0].x, S[j][0].y);
                x.y = StateIO<true>::pack(S[j][0].z, S[j][0].w);
                x.z = StateIO<true>::pack(S[j][1].x, S[j][1].y);
                x.w = StateIO<true>::pack(S[j][1].z, S[j][1].w);
            } else {
                x = __builtin_bit_cast(u4, S[j][0]);
            }
            store_b128(x, dst, lane_off, (8 * wave + RPI * j) * row_bytes);
        }
    }
}

struct ReplayParams {
    int32_t B, T, HV;
    int32_t xcd_block;
    const float *factors;
    void *pool;
    int64_t sp_slot, sp_head, sp_row;
    const int32_t *ridx;
    const int32_t *widx;
    const int32_t *ntok;
    const int32_t *cu;  // varlen token offsets, or null
    int32_t total;
};

// Rebuild the state of (request, value head) from its update records:
// S <- S diag(a_t) + err_t k_t^T for t < ntok. Same tile mapping as the
// decode kernel; the records of up to 8 tokens are staged in LDS.
template <int K, int V, bool BF16S>
__global__ void __launch_bounds__((V / kRowsPerWave) * 64)
replay_kernel(const ReplayParams p)
{
    using IO = StateIO<BF16S>;
    constexpr uint32_t ES = IO::ES;
    constexpr int NW = V / kRowsPerWave;
    constexpr int RPL = kRowsPerWave / 8;
    constexpr int CPL = K / 32;
    constexpr int RS = 2 * K + V;  // floats per record
    __shared__ f4 recs[kTokChunk * RS / 4];
    const float *lrec = reinterpret_cast<const float *>(recs);

    const int pair = pair_of_block(p.xcd_block);
    const int b = pair / p.HV;
    const int hv = pair - b * p.HV;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c8 = lane & 7;
    const int rs = lane >> 3;
    const int r = __builtin_amdgcn_readfirstlane(p.ridx[b]);
    const int w = __builtin_amdgcn_readfirstlane(p.widx ? p.widx[b] : r);
    const int n = __builtin_amdgcn_readfirstlane(p.ntok[b]);
    int Tb, tok0;
    int64_t flat0;
    if (!request_tokens(p.cu, p.total, b, p.T, Tb, tok0, flat0))
        return;
    if (r < 0 || n < 0 || n > Tb)
        return;

    const uint32_t row_bytes = static_cast<uint32_t>(p.sp_row) * ES;
    const uint32_t tile_bytes = static_cast<uint32_t>(
        (static_cast<int64_t>(V - 1) * p.sp_row + K) * ES);
    const uint32_t lane_off = rs * row_bytes + c8 * 16u;
    char *const pool = static_cast<char *>(p.pool);
    const BufRsrc src = make_rsrc(
        pool + (r * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
    f4 S[RPL][CPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        IO::template load_row<kStreamPolicy>(
            S[i], src, lane_off, (wave * kRowsPerWave + i * 8) * row_bytes);

    const f4 *grec = reinterpret_cast<const f4 *>(
        p.factors + (flat0 * p.HV + hv) * RS);
    const int64_t tstride4 = static_cast<int64_t>(p.HV) * RS / 4;
    for (int t0 = 0; t0 < n; t0 += kTokChunk) {
        const int nt = min(kTokChunk, n - t0);
        if (t0 > 0)
            lds_barrier();
        for (int i = threadIdx.x; i < nt * (RS / 4); i += NW * 64) {
            const int tt = i / (RS / 4), e = i - tt * (RS / 4);
            recs[i] = grec[(t0 + tt) * tstride4 + e];
        }
        lds_barrier();
        for (int tt = 0; tt < nt; ++tt) {
            const float *rec = lrec + tt * RS;
            float err[RPL];
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                err[i] = rec[2 * K + wave * kRowsPerWave + i * 8 + rs];
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const f4 a = *reinterpret_cast<const f4 *>(
                    rec + IO::col(m, c8));
                const f4 kk = *reinterpret_cast<const f4 *>(
                    rec + K + IO::col(m, c8));
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    S[i][m] *= a;
                    S[i][m].x = fmaf(err[i], kk.x, S[i][m].x);
                    S[i][m].y = fmaf(err[i], kk.y, S[i][m].y);
                    S[i][m].z = fmaf(err[i], kk.z, S[i][m].z);
                    S[i][m].w = fmaf(err[i], kk.w, S[i][m].w);
                }
            }
        }
    }

    if (w >= 0) {
        const BufRsrc dst = make_rsrc(
            pool + (w * p.sp_slot + hv * p.sp_head) * ES, tile_bytes);
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            IO::store_row(dst, lane_off,
                          (wave * kRowsPerWave + i * 8) * row_bytes, S[i]);
    }
}

// Validators of the device preconditions. A one-thread kernel clears the
// result word (a kernel rather than a memset, so that the call can be
// captured into a graph), then the checking grid runs one workgroup per
// request, which compares that request with every other one and ORs what it
// finds into the word: the quadratic scan is spread over B workgroups.
constexpr int kCheckThreads = 256;

__global__ void __launch_bounds__(64) clear_result_kernel(int32_t *result)
{
    if (threadIdx.x == 0)
        *result = 0;
}

// OR of the workgroup's flags into *result: one global atomic per
// workgroup that found something.
__device__ __forceinline__ void or_flags(int32_t f, int32_t *result)
{
    __shared__ int32_t flags;
    if (threadIdx.x == 0)
        flags = 0;
    __syncthreads();
    if (f)
        atomicOr(&flags, f);
    __syncthreads();
    if (threadIdx.x == 0 && flags)
        atomicOr(result, flags);
}

// Request i = blockIdx.x against every request j != i.
__global__ void __launch_bounds__(kCheckThreads)
check_indices_kernel(int32_t B, int32_t pool_size, const int32_t *ridx,
                     const int32_t *widx, int32_t *result)
{
    const int i = blockIdx.x;
    const int32_t r = ridx[i];
    const int32_t w = widx ? widx[i] : r;
    int32_t f = 0;
    if (threadIdx.x == 0) {
        if (r >= pool_size)
            f |= 1;
        if (r >= 0 && w >= pool_size)
            f |= 2;
    }
    if (r >= 0 && w >= 0) {
        for (int j = threadIdx.x; j < B; j += kCheckThreads) {
            if (j == i)
                continue;
            const int32_t rj = ridx[j];
            if (rj < 0)
                continue;
            const int32_t wj = widx ? widx[j] : rj;
            if (wj == w)
                f |= 4;
            if (rj == w)
                f |= 8;
        }
    }
    or_flags(f, result);
}

// Paged per-token slot table: request i = blockIdx.x; its seed and table
// entries against every active request j != i.
__global__ void __launch_bounds__(kCheckThreads)
check_token_slots_kernel(int32_t B, int32_t T, int32_t pool_size,
                         const int32_t *tab, int64_t stride,
                         const int32_t *nacc, int32_t *result)
{
    const int i = blockIdx.x;
    const int32_t *row = tab + i * stride;
    const int32_t na = nacc[i];
    int32_t f = 0;
    if (na < 1 || na > T) {
        if (threadIdx.x == 0)
            f |= 16;
    } else {
        const int32_t seed = row[na - 1];
        if (threadIdx.x == 0 && seed >= pool_size)
            f |= 1;
        if (seed >= 0) {
            for (int t = threadIdx.x; t < T; t += kCheckThreads)
                if (row[t] >= pool_size)
                    f |= 2;
            for (int j = threadIdx.x; j < B; j += kCheckThreads) {
                if (j == i)
                    continue;
                const int32_t nj = nacc[j];
                if (nj < 1 || nj > T)
                    continue;
                const int32_t *rowj = tab + j * stride;
                const int32_t sj = rowj[nj - 1];
                if (sj < 0)
                    continue;
                for (int t = 0; t < T; ++t) {
                    const int32_t s = row[t];
                    if (s < 0)
                        continue;
                    if (sj == s)
                        f |= 8;
                    for (int u = 0; u < T; ++u)
                        if (rowj[u] == s)
                            f |= 4;
                }
            }
        }
    }
    or_flags(f, result);
}

// Validator of varlen offsets (one workgroup): bit 1 = an offset outside
// [0, total], bit 2 = a request with a negative count or more than T tokens.
__global__ void __launch_bounds__(1024)
check_cu_seqlens_kernel(int32_t B, int32_t T, int32_t total,
                        const int32_t *cu, int32_t *result)
{
    __shared__ int32_t flags;
    if (threadIdx.x == 0)
        flags = 0;
    __syncthreads();
    int32_t f = 0;
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
        const int32_t c0 = cu[i], c1 = cu[i + 1];
        if (c0 < 0 || c0 > total || c1 < 0 || c1 > total)
            f |= 1;
        if (c1 < c0 || c1 - c0 > T)
            f |= 2;
    }
    if (f)
        atomicOr(&flags, f);
    __syncthreads();
    if (threadIdx.x == 0)
        *result = flags;
}

// ------------------------------------------------------------- host side

typedef void (*KernelFn)(const Params);

// A decode_kernel instance: its entry, its rows per wave (the workgroup has
// V / rows waves) and its tokens per LDS round (CH; the launch's LDS is
// min(T, CH) token records). The launch shape is read from here, so it
// always matches the instance that runs.
struct Instance {
    KernelFn fn;
    int rows;
    int ch;
    int stage_floats;  // LDS beyond the token records (staged write-back)
};

template <int VAR, int K, int V, bool BF16S, bool REC, int R, int CH>
Instance pick_io(bool bf16_in, bool bf16_out)
{
    KernelFn fn;
    if (bf16_in)
        fn = bf16_out
                 ? decode_kernel<VAR, K, V, true, true, BF16S, REC, R, CH>
                 : decode_kernel<VAR, K, V, true, false, BF16S, REC, R, CH>;
    else
        fn = bf16_out
                 ? decode_kernel<VAR, K, V, false, true, BF16S, REC, R, CH>
                 : decode_kernel<VAR, K, V, false, false, BF16S, REC, R, CH>;
    // LDS of the staged write-back (fp32 outputs only)
    constexpr int stage = staged_writeback<K, V, false, BF16S, REC, R, CH>()
                              ? (V / R) * 8 * kStageRowFloats
                              : 0;
    return {fn, R, CH, bf16_out ? 0 : stage};
}

// ch: the tokens per round the call asks for (kTokChunk, kKdaTokChunk or
// kCacheTokChunk); records and small grids always take kTokChunk.
template <int VAR, int K, int V>
Instance pick_dtype(bool bf16_in, bool bf16_out, bool bf16_state, bool rec,
                    bool small, int ch)
{
    constexpr int RR = kRecordRowsPerWave, RS = kSmallGridRowsPerWave;
    constexpr int RP = kRowsPerWave;
    constexpr int C8 = kTokChunk, C4 = kKdaTokChunk, C2 = kCacheTokChunk;
    const bool bi = bf16_in, bo = bf16_out;
    if (rec)
        return bf16_state ? pick_io<VAR, K, V, true, true, RR, C8>(bi, bo)
                          : pick_io<VAR, K, V, false, true, RR, C8>(bi, bo);
    if (small)
        return bf16_state ? pick_io<VAR, K, V, true, false, RS, C8>(bi, bo)
                          : pick_io<VAR, K, V, false, false, RS, C8>(bi, bo);
    if constexpr (V == 128)
        if (ch == C2)
            return bf16_state
                       ? pick_io<VAR, K, V, true, false, RP, C2>(bi, bo)
                       : pick_io<VAR, K, V, false, false, RP, C2>(bi, bo);
    if constexpr (VAR == VAR_KDA)
        if (ch == C4)
            return bf16_state
                       ? pick_io<VAR, K, V, true, false, RP, C4>(bi, bo)
                       : pick_io<VAR, K, V, false, false, RP, C4>(bi, bo);
    return bf16_state ? pick_io<VAR, K, V, true, false, RP, C8>(bi, bo)
                      : pick_io<VAR, K, V, false, false, RP, C8>(bi, bo);
}

template <int VAR, int K, int V>
KernelFn pick_packed(bool bi, bool bo)
{
    if (bi)
        return bo ? decode_packed_kernel<VAR, K, V, true, true>
                  : decode_packed_kernel<VAR, K, V, true, false>;
    return bo ? decode_packed_kernel<VAR, K, V, false, true>
              : decode_packed_kernel<VAR, K, V, false, false>;
}

template <int VAR>
KernelFn pick_packed(int K, int V, bool bi, bool bo)
{
    if (K == 128)
        return V == 128 ? pick_packed<VAR, 128, 128>(bi, bo)
                        : pick_packed<VAR, 128, 64>(bi, bo);
    return V == 128 ? pick_packed<VAR, 64, 128>(bi, bo)
                    : pick_packed<VAR, 64, 64>(bi, bo);
}

template <int VAR, int K, int V, bool BF16S>
KernelFn pick_one(bool bi, bool bo)
{
    if (bi)
        return bo ? decode1_kernel<VAR, K, V, true, true, BF16S>
                  : decode1_kernel<VAR, K, V, true, false, BF16S>;
    return bo ? decode1_kernel<VAR, K, V, false, true, BF16S>
              : decode1_kernel<VAR, K, V, false, false, BF16S>;
}

template <int VAR, int K, int V>
KernelFn pick_one(bool bi, bool bo, bool bs)
{
    return bs ? pick_one<VAR, K, V, true>(bi, bo)
              : pick_one<VAR, K, V, false>(bi, bo);
}

template <int VAR>
KernelFn pick_one(int K, int V, bool bi, bool bo, bool bs)
{
    if (K == 128)
        return V == 128 ? pick_one<VAR, 128, 128>(bi, bo, bs)
                        : pick_one<VAR, 128, 64>(bi, bo, bs);
    return V == 128 ? pick_one<VAR, 64, 128>(bi, bo, bs)
                    : pick_one<VAR, 64, 64>(bi, bo, bs);
}

template <int VAR>
Instance pick(int K, int V, bool bi, bool bo, bool bs, bool rec, bool small,
              int ch)
{
    if (K == 128)
        return V == 128
                   ? pick_dtype<VAR, 128, 128>(bi, bo, bs, rec, small, ch)
                   : pick_dtype<VAR, 128, 64>(bi, bo, bs, rec, small, ch);
    return V == 128 ? pick_dtype<VAR, 64, 128>(bi, bo, bs, rec, small, ch)
                    : pick_dtype<VAR, 64, 64>(bi, bo, bs, rec, small, ch);
}

int lds_floats_per_token(int var, int K, int V)
{
    return (var == VAR_KDA ? 3 : 2) * K + V + 4;
}

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

bool strides_nonneg(const la_act_strides &s)
{
    return s.b >= 0 && s.t >= 0 && s.h >= 0;
}

// Whether every element offset of an activation tensor [nb, nt, nh, inner]
// (strides s, innermost stride 1) fits in 31 bits.
bool fits31(const la_act_strides &s, int64_t nb, int64_t nt, int64_t nh,
            int64_t inner)
{
    if (nb < 1 || nt < 1 || nh < 1)
        return true;  // nothing is indexed
    const int64_t st[3] = {s.b, s.t, s.h};
    const int64_t ex[3] = {nb - 1, nt - 1, nh - 1};
    int64_t off = inner - 1;
    for (int i = 0; i < 3; ++i) {
        if (ex[i] == 0)
            continue;
        if (st[i] > INT32_MAX || ex[i] > INT32_MAX)
            return false;
        off += st[i] * ex[i];  // each term < 2^62, at most three of them
        if (off > INT32_MAX)
            return false;
    }
    return off <= INT32_MAX;
}

// True when the n blocks (extent[i] copies at stride[i]) of `inner`
// contiguous elements never overlap: sorted by stride, each stride must
// clear everything nested inside it.
bool no_overlap(int n, const int64_t *stride, const int64_t *extent,
                int64_t inner)
{
    int order[4];
    for (int i = 0; i < n; ++i)
        order[i] = i;
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && stride[order[j]] < stride[order[j - 1]]; --j) {
            const int tmp = order[j];
            order[j] = order[j - 1];
            order[j - 1] = tmp;
        }
    int64_t span = inner;  // elements covered by the dims processed so far
    for (int i = 0; i < n; ++i) {
        const int d = order[i];
        if (extent[d] <= 1)
            continue;
        if (stride[d] < span)
            return false;
        span = stride[d] * (extent[d] - 1) + span;
    }
    return true;
}

la_status validate(const la_decode_args *a, int var)
{
    if (!a)
        return LA_ERR_NULL;
    if (a->B < 0 || a->T < 1 || a->H < 1 || a->HV < 1 || a->pool_size < 1)
        return LA_ERR_SHAPE;
    if (a->HV % a->H != 0)
        return LA_ERR_SHAPE;
    if ((a->K != 64 && a->K != 128) || (a->V != 64 && a->V != 128))
        return LA_ERR_UNSUPPORTED;
    if ((a->qkv_dtype != LA_F32 && a->qkv_dtype != LA_BF16) ||
        (a->out_dtype != LA_F32 && a->out_dtype != LA_BF16) ||
        (a->state_dtype != LA_F32 && a->state_dtype != LA_BF16))
        return LA_ERR_DTYPE;
    if (a->reserved != 0 || a->reserved2 != 0)
        return LA_ERR_ARG;
    if (a->cu_seqlens && a->total_tokens < 0)
        return LA_ERR_SHAPE;
    if (var == VAR_LA) {
        if (a->flags != 0 || a->beta != nullptr || a->A_log || a->dt_bias)
            return LA_ERR_ARG;
    } else {
        if (a->flags & ~(LA_F_L2NORM_QK | LA_F_BETA_LOGIT | LA_F_GATE |
                         LA_F_GATE_LOWER_BOUND))
            return LA_ERR_ARG;
        const bool gate = (a->flags & LA_F_GATE) != 0;
        // gate inputs without the switch are refused, not ignored
        if (!gate && (a->A_log || a->dt_bias ||
                      (a->flags & LA_F_GATE_LOWER_BOUND)))
            return LA_ERR_ARG;
        if ((a->flags & LA_F_GATE_LOWER_BOUND) &&
            !(a->lower_bound < 0.f && a->lower_bound > -3.0e38f))
            return LA_ERR_ARG;
        if (gate && a->B > 0 && (!a->A_log || !a->dt_bias))
            return LA_ERR_NULL;
    }
    if (static_cast<int64_t>(a->B) * a->HV > INT32_MAX)
        return LA_ERR_SHAPE;
    if (a->B == 0)
        return LA_OK;

    if (a->token_slots) {
        // paged mode: the table replaces the read/write slot arrays
        if (a->read_idx || a->write_idx)
            return LA_ERR_ARG;
        if (!a->num_accepted)
            return LA_ERR_NULL;
        if (a->token_slots_stride < a->T)
            return LA_ERR_STRIDE;
        if (!aligned(a->token_slots, 4) || !aligned(a->num_accepted, 4))
            return LA_ERR_ALIGN;
    } else {
        if (!a->read_idx)
            return LA_ERR_NULL;
        if (a->num_accepted)
            return LA_ERR_ARG;
    }
    // A token-packed batch of no tokens indexes no per-token array (the
    // kernels skip any request whose offsets pass total_tokens), so its
    // empty q, k, v, g, beta and out may come without an address.
    const bool no_tokens = a->cu_seqlens && a->total_tokens == 0;
    if (!a->pool || (!no_tokens && (!a->q || !a->k || !a->v || !a->out)))
        return LA_ERR_NULL;
    if (var != VAR_LA && !no_tokens && (!a->g || !a->beta))
        return LA_ERR_NULL;

    if (!strides_nonneg(a->sq) || !strides_nonneg(a->sk) ||
        !strides_nonneg(a->sv) || !strides_nonneg(a->so))
        return LA_ERR_STRIDE;
    if (var != VAR_LA && (!strides_nonneg(a->sg) || !strides_nonneg(a->sbeta)))
        return LA_ERR_STRIDE;
    {
        // 32-bit activation offsets (per-request b strides unused when
        // the batch is token-packed)
        const int64_t nb = a->cu_seqlens ? 1 : a->B;
        const int64_t nt = a->cu_seqlens ? a->total_tokens : a->T;
        if (!fits31(a->sq, nb, nt, a->H, a->K) ||
            !fits31(a->sk, nb, nt, a->H, a->K) ||
            !fits31(a->sv, nb, nt, a->HV, a->V) ||
            !fits31(a->so, nb, nt, a->HV, a->V))
            return LA_ERR_STRIDE;
        if (var != VAR_LA &&
            (!fits31(a->sg, nb, nt, a->HV, var == VAR_KDA ? a->K : 1) ||
             !fits31(a->sbeta, nb, nt, a->HV, 1)))
            return LA_ERR_STRIDE;
    }
    if (a->sp.slot < 0 || a->sp.head < 0 || a->sp.row < 0)
        return LA_ERR_STRIDE;

    // pool tiles: rows K wide inside a tile, tiles disjoint
    {
        const int64_t st[3] = {a->sp.row, a->sp.head, a->sp.slot};
        const int64_t ex[3] = {a->V, a->HV, a->pool_size};
        if (!no_overlap(3, st, ex, a->K))
            return LA_ERR_STRIDE;
    }
    // a tile is addressed with 32-bit byte offsets from its first row
    const int64_t es = a->state_dtype == LA_BF16 ? 2 : 4;
    if ((static_cast<int64_t>(a->V - 1) * a->sp.row + a->K) * es > INT32_MAX)
        return LA_ERR_STRIDE;
    // outputs must not overlap each other ([total, HV, V] when varlen)
    if (a->cu_seqlens) {
        const int64_t st[2] = {a->so.h, a->so.t};
        const int64_t ex[2] = {a->HV, a->total_tokens};
        if (!no_overlap(2, st, ex, a->V))
            return LA_ERR_STRIDE;
    } else {
        const int64_t st[3] = {a->so.h, a->so.t, a->so.b};
        const int64_t ex[3] = {a->HV, a->T, a->B};
        if (!no_overlap(3, st, ex, a->V))
            return LA_ERR_STRIDE;
    }

    const uintptr_t act = a->qkv_dtype == LA_BF16 ? 2 : 4;
    const uintptr_t outsz = a->out_dtype == LA_BF16 ? 2 : 4;
    if (!aligned(a->q, act) || !aligned(a->k, act) || !aligned(a->v, act) ||
        !aligned(a->out, outsz) || !aligned(a->read_idx, 4) ||
        !aligned(a->write_idx, 4))
        return LA_ERR_ALIGN;
    if (a->g && !aligned(a->g, 4))
        return LA_ERR_ALIGN;
    if (a->beta && !aligned(a->beta, 4))
        return LA_ERR_ALIGN;
    // lanes move 16-byte chunks: every row start 16-byte aligned
    const int64_t epc = 16 / es;  // elements per chunk
    if (!aligned(a->pool, 16) || (a->sp.slot % epc) || (a->sp.head % epc) ||
        (a->sp.row % epc))
        return LA_ERR_ALIGN;
    if (a->inter && !aligned(a->inter, 16))
        return LA_ERR_ALIGN;
    if (a->factors && !aligned(a->factors, 16))
        return LA_ERR_ALIGN;
    if (!aligned(a->cu_seqlens, 4) || !aligned(a->A_log, 4) ||
        !aligned(a->dt_bias, 4))
        return LA_ERR_ALIGN;
    return LA_OK;
}

// Pairs per XCD block for a grid of B * HV pairs. Below 48 value heads one
// contiguous range per XCD (whole requests on one XCD); from 48 heads blocks
// of 32 pairs. Measured on MI355X against the plain order (each XCD takes
// every eighth pair), % of peak HBM bandwidth:
//   ranges, < 48 heads: KDA B=256 H=24 70.7 -> 72.3; GDN B=256 HV=32
//   71.3 -> 73.2; GDN B=32 T=4 with the cache 65.9 -> 67.4; paged GDN B=64
//   T=4 65.1 -> 67.2; one-token GDN B=64 HV=32 69.1 -> 70.3 (four slot
//   draws: +0.3 to +1.9); bf16 one-token GDN HV=16..32 +2.3 to +2.7.
//   Ranges at 64 heads lose (GDN HV=64 T=2 73.2 -> 69.3; one-token
//   Lightning H=64 74.6 -> 68.8).
//   32-pair blocks, >= 48 heads: Lightning B=33 H=64 74.0 -> 75.1; GDN
//   HV=48 71.8 -> 72.7, HV=96 74.6 -> 76.1; Lightning K=V=64 H=64 71.1 ->
//   74.2; GDN HV=64 T=2 and Lightning H=64 B=64 unchanged.
// Dense KDA calls of more than four tokens with no per-token writes (four
// tokens per LDS round) keep the plain order: same boxes, 4 GiB rotation,
// steady clocks, us per call, ranges -> plain: KDA B=256 H=24 T=8 163.2 ->
// 161.3 (three boxes, 1.0-1.1 %), B=128 T=8 88.5 -> 87.1, bf16 pool B=128
// T=8 66.3 -> 64.9, B=96 H=8 T=8 26.7 -> 26.5, B=64 T=16 71.4 -> 71.0; T=6
// and K = V = 64 even, T=5 143.9 -> 144.2. Varlen KDA batches keep ranges
// (B=128 T<=8: 77.6 -> 78.0), and so do the calls that write a state per
// token, where the plain order loses 2-4 % (GDN B=32 T=4 with the cache
// 69.1 -> 70.5, paged GDN B=64 T=4 121.7 -> 126.7, KDA B=64 T=4 with the
// cache 112.7 -> 116.0), and the K = V = 64 one-token grids (GDN B=256
// HV=32: 46.2 -> 52.7).
// The packed kernel keeps the plain order (13 bf16 shapes: -2.5 to +2.7),
// and so does the small-grid instance, where ranges lost up to 4.5 points
// (GDN B=32 HV=16 T=4 with the cache, 512 tiles: 66.6 -> 62.1; GDN B=64
// HV=8: 66.7 -> 64.8).
int xcd_block_for(int B, int HV)
{
    const int64_t n = static_cast<int64_t>(B) * HV;
    if (HV >= kXcdRangeMaxHeads)
        return kXcdBlockPairs;
    return n >= 16 ? static_cast<int>(n / 8) : 1;
}

// The kernel, launch shape and parameters of a decode call. fn is null
// when there is nothing to launch (B = 0).
struct Launch {
    KernelFn fn = nullptr;
    const char *name = "none";
    dim3 grid, block;
    size_t lds = 0;
    int ch = 0;  // tokens per LDS round of the instance
    Params p;
};

// Host checks, kernel choice and parameter block of a decode call.
la_status select_kernel(const la_decode_args *a, int var, Launch &L)
{
    const la_status st = validate(a, var);
    if (st != LA_OK || a->B == 0)
        return st;

    Params &p = L.p;
    p.B = a->B;
    p.T = a->T;
    p.HV = a->HV;
    p.group = a->HV / a->H;
    p.flags = a->flags;
    p.q = a->q;
    p.sq_b = a->sq.b;
    p.sq_t = a->sq.t;
    p.sq_h = a->sq.h;
    p.k = a->k;
    p.sk_b = a->sk.b;
    p.sk_t = a->sk.t;
    p.sk_h = a->sk.h;
    p.v = a->v;
    p.sv_b = a->sv.b;
    p.sv_t = a->sv.t;
    p.sv_h = a->sv.h;
    p.g = a->g;
    p.sg_b = a->sg.b;
    p.sg_t = a->sg.t;
    p.sg_h = a->sg.h;
    p.beta = a->beta;
    p.sb_b = a->sbeta.b;
    p.sb_t = a->sbeta.t;
    p.sb_h = a->sbeta.h;
    p.pool = a->pool;
    p.sp_slot = a->sp.slot;
    p.sp_head = a->sp.head;
    p.sp_row = a->sp.row;
    p.ridx = a->read_idx;
    p.widx = a->write_idx;
    p.inter = a->inter;
    p.out = a->out;
    p.so_b = a->so.b;
    p.so_t = a->so.t;
    p.so_h = a->so.h;
    p.tslots = a->token_slots;
    p.ts_stride = a->token_slots_stride;
    p.naccept = a->num_accepted;
    p.factors = a->factors;
    p.cu = a->cu_seqlens;
    p.total = a->cu_seqlens ? a->total_tokens : 0;
    p.gate = !(a->flags & LA_F_GATE)            ? 0
             : (a->flags & LA_F_GATE_LOWER_BOUND) ? 2
                                                 : 1;
    p.A_log = a->A_log;
    p.dt_bias = a->dt_bias;
    p.lower_bound = a->lower_bound;
    if (a->cu_seqlens) {
        // token-packed arrays: the flat token number goes through the t
        // strides, so the per-request strides drop out
        p.sq_b = p.sk_b = p.sv_b = p.sg_b = p.sb_b = p.so_b = 0;
    }

    const bool bi = a->qkv_dtype == LA_BF16, bo = a->out_dtype == LA_BF16;
    const bool bs = a->state_dtype == LA_BF16;
    const bool rec = a->factors != nullptr;
    // One token with no per-token writes: the contiguous-row kernel where
    // it is the faster one. All three kernels give identical bits, so the
    // choice is by speed alone. Measured on MI355X at steady clocks with a
    // 4 GiB rotation (the one-token kernel in 4 workgroups per tile),
    // general -> one-token kernel, us per call:
    //   fp32 K = V = 128 beyond 1024 tiles (one resident round of the
    //   general kernel), any head count: 1032-1536 tiles: KDA H=24 B=43
    //   26.8 -> 25.1, B=64 37.5 -> 35.1; KDA H=12 B=128 38.1 -> 36.9; GDN
    //   HV=32 B=48 37.4 -> 34.6; GDN HV=16 B=96 37.6 -> 35.8; Lightning
    //   H=32 B=33 27.8 -> 24.7, B=48 37.4 -> 34.2; Lightning H=16 B=96 37.3
    //   -> 35.1; 2048 tiles and more: GDN B=64 HV=32 48.3 -> 45.3; GDN
    //   HV=16 B=256 97.8 -> 95.5; HV=24 B=256 141.4 -> 136.7; HV=32 B=256
    //   184.9 -> 178.1; Lightning H=16 B=256 96.5 -> 92.5; KDA H=24 B=96
    //   55.4 -> 52.3, B=256 141.2 -> 136.6
    //   exactly 1024 tiles: Lightning H=64 B=16 24.4 -> 23.1 (48 or more
    //   heads take it), but GDN HV=32 B=32 24.0 -> 24.2 and HV=16 B=64 24.8
    //   -> 25.6; 512-768 tiles: the general kernel (Lightning H=16 B=32
    //   12.7 against 13.8, KDA H=3 B=256 18.0 against 20.3)
    //   K = V = 64: 2048 tiles 12.8 -> 14.4; 8192 tiles: GDN 51.5 -> 46.2,
    //   KDA 51.4 -> 46.6
    // On a bf16 pool the packed kernel keeps the grids it runs in one
    // resident round: 2048 tiles for Lightning and GDN (4 waves per SIMD),
    // 1536 for KDA (142 VGPRs, 3 waves per SIMD). Packed against one-token
    // kernel: GDN HV=32 1024 tiles 13.2 against 14.3, 1536 tiles 19.1
    // against 19.5, 2048 tiles 25.0 against 24.7 (HV=16: 25.5 against
    // 26.0); KDA H=24 1536 tiles 19.1 against 20.2, 1920 tiles 27.2
    // against 23.9. Beyond, the one-token kernel: KDA H=24 B=96 32.3 ->
    // 28.1 and B=128 41.2 -> 37.3 (packed), B=256 76.5 -> 72.7 (general).
    const int64_t tiles = static_cast<int64_t>(a->B) * a->HV;
    const bool wide = a->K == 128 && a->V == 128
                          ? tiles > 1024 || (a->HV >= 48 && tiles == 1024)
                          : tiles >= 4096;
    const int64_t packed_max = var == VAR_KDA ? kPackedMaxTilesKda
                                              : kPackedMaxTiles;
    const bool one = a->T == 1 && !a->inter && !a->token_slots && !rec &&
                     !a->cu_seqlens && (bs ? tiles > packed_max : wide);
    // otherwise one token on a bf16 pool with no per-token writes (up to
    // packed_max tiles): the packed tile
    const bool packed = !one && bs && a->T == 1 && !a->inter &&
                        !a->token_slots && !rec && !a->cu_seqlens;
    // a grid of the general kernel that fills less than one resident round
    const bool small = !packed && !one && !rec &&
                       tiles * (a->V / kSmallGridRowsPerWave) <= kSmallGridWaves;
    // other grids that write a state per token stage kCacheTokChunk tokens
    // per LDS round (at V = 128: at V = 64 the KDA instance would need 129
    // VGPRs, one wave per SIMD less)
    const bool cache = !packed && !one && !rec && !small && a->V == 128 &&
                       !a->cu_seqlens && (a->inter || a->token_slots);
    // tokens per LDS round asked of the general kernel
    const bool kda_mid = var == VAR_KDA && !packed && !one && !rec &&
                         !small && !cache && !a->inter && !a->token_slots &&
                         a->T > kKdaTokChunk;
    const int ch = cache ? kCacheTokChunk
                   : kda_mid ? kKdaTokChunk
                             : kTokChunk;
    // rows per wave and tokens per round of the instance that runs: 64 rows
    // and one token in the packed kernel, 8 rows and no LDS in the one-token
    // kernel
    Instance inst;
    if (packed)
        inst = {var == VAR_LA    ? pick_packed<VAR_LA>(a->K, a->V, bi, bo)
                : var == VAR_GDN ? pick_packed<VAR_GDN>(a->K, a->V, bi, bo)
                                 : pick_packed<VAR_KDA>(a->K, a->V, bi, bo),
                64, 1, 0};
    else if (one)
        inst = {var == VAR_LA    ? pick_one<VAR_LA>(a->K, a->V, bi, bo, bs)
                : var == VAR_GDN ? pick_one<VAR_GDN>(a->K, a->V, bi, bo, bs)
                                 : pick_one<VAR_KDA>(a->K, a->V, bi, bo, bs),
                8, 0, 0};
    else
        inst = var == VAR_LA
                   ? pick<VAR_LA>(a->K, a->V, bi, bo, bs, rec, small, ch)
               : var == VAR_GDN
                   ? pick<VAR_GDN>(a->K, a->V, bi, bo, bs, rec, small, ch)
                   : pick<VAR_KDA>(a->K, a->V, bi, bo, bs, rec, small, ch);
    // the packed kernel and the small-grid instance keep the plain order;
    // the one-token kernel at K = V = 128 splits tiles and deals blocks of
    // kOneXcdTiles whole tiles to the XCDs in turn
    p.split_log2 = one && a->K == 128 && a->V == 128 ? kOneSplitLog2 : 0;
    // dense KDA calls of more than kKdaTokChunk tokens without per-token
    // writes keep the plain order (see xcd_block_for)
    const bool plain = packed || small || (kda_mid && !a->cu_seqlens);
    p.xcd_block = p.split_log2 ? kOneXcdTiles << p.split_log2
                  : plain      ? 1
                               : xcd_block_for(a->B, a->HV);
    L.fn = inst.fn;
    L.name = packed ? "decode_packed_kernel"
             : one  ? "decode1_kernel"
                    : "decode_kernel";
    L.ch = inst.ch;
    const int chunk = a->T < inst.ch ? a->T : inst.ch;
    L.lds = (static_cast<size_t>(chunk) *
                 lds_floats_per_token(var, a->K, a->V) +
             inst.stage_floats) *
            sizeof(float);
    L.grid = dim3((static_cast<unsigned>(a->B) * a->HV) << p.split_log2);
    L.block = dim3(((a->V / inst.rows) * 64) >> p.split_log2);
    return LA_OK;
}

la_status launch(const la_decode_args *a, void *stream, int var)
{
    Launch L;
    const la_status st = select_kernel(a, var, L);
    if (st != LA_OK || !L.fn)
        return st;
    void *kargs[] = {&L.p};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(L.fn), L.grid, L.block, kargs, L.lds,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

// The clearing kernel, then (B > 0) the checking grid of B workgroups.
la_status launch_check(const void *kernel, int32_t B, void **kargs,
                       int32_t *dev_result, void *stream)
{
    const hipStream_t st = static_cast<hipStream_t>(stream);
    void *cargs[] = {&dev_result};
    hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(clear_result_kernel), dim3(1),
        dim3(64), cargs, 0, st);
    if (e == hipSuccess && B > 0)
        e = hipLaunchKernel(kernel, dim3(static_cast<unsigned>(B)),
                            dim3(kCheckThreads), kargs, 0, st);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

la_status la_decode_kernel_info(int32_t variant, const la_decode_args *args,
                                la_kernel_info *info)
{
    if (!info)
        return LA_ERR_NULL;
    if (variant != LA_VARIANT_LIGHTNING && variant != LA_VARIANT_GDN &&
        variant != LA_VARIANT_KDA)
        return LA_ERR_ARG;
    static_assert(static_cast<int>(LA_VARIANT_LIGHTNING) == VAR_LA &&
                      static_cast<int>(LA_VARIANT_GDN) == VAR_GDN &&
                      static_cast<int>(LA_VARIANT_KDA) == VAR_KDA,
                  "variant codes");
    Launch L;
    const la_status st = select_kernel(args, variant, L);
    if (st != LA_OK)
        return st;
    la_kernel_info r = {};
    r.kernel = L.name;
    if (L.fn) {
        hipFuncAttributes at;
        int nb = 0;
        const void *f = reinterpret_cast<const void *>(L.fn);
        if (hipFuncGetAttributes(&at, f) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &nb, f, static_cast<int>(L.block.x), L.lds) != hipSuccess)
            return LA_ERR_LAUNCH;
        r.grid_blocks = static_cast<int32_t>(L.grid.x);
        r.block_threads = static_cast<int32_t>(L.block.x);
        r.lds_bytes = static_cast<int32_t>(L.lds);
        r.vgprs = at.numRegs;
        r.scratch_bytes = static_cast<int32_t>(at.localSizeBytes);
        r.blocks_per_cu = nb;
        r.waves_per_simd = nb * static_cast<int32_t>(L.block.x / 64) / 4;
        r.tokens_per_round = L.ch;
    }
    *info = r;
    return LA_OK;
}

la_status la_decode(const la_decode_args *args, void *stream)
{
    return launch(args, stream, VAR_LA);
}

la_status gdn_decode_mtp(const la_decode_args *args, void *stream)
{
    return launch(args, stream, VAR_GDN);
}

la_status kda_decode_mtp(const la_decode_args *args, void *stream)
{
    return launch(args, stream, VAR_KDA);
}

la_status la_replay(const la_replay_args *a, void *stream)
{
    if (!a)
        return LA_ERR_NULL;
    if (a->B < 0 || a->T < 1 || a->HV < 1 || a->pool_size < 1)
        return LA_ERR_SHAPE;
    if ((a->K != 64 && a->K != 128) || (a->V != 64 && a->V != 128))
        return LA_ERR_UNSUPPORTED;
    if (a->state_dtype != LA_F32 && a->state_dtype != LA_BF16)
        return LA_ERR_DTYPE;
    if (a->reserved != 0)
        return LA_ERR_ARG;
    if (a->cu_seqlens && a->total_tokens < 0)
        return LA_ERR_SHAPE;
    if (static_cast<int64_t>(a->B) * a->HV > INT32_MAX)
        return LA_ERR_SHAPE;
    if (a->B == 0)
        return LA_OK;
    // no records to read in a token-packed batch of no tokens (a request
    // asking for more records than its tokens is skipped)
    const bool no_tokens = a->cu_seqlens && a->total_tokens == 0;
    if ((!a->factors && !no_tokens) || !a->pool || !a->read_idx ||
        !a->num_tokens)
        return LA_ERR_NULL;
    if (!aligned(a->cu_seqlens, 4))
        return LA_ERR_ALIGN;
    if (a->sp.slot < 0 || a->sp.head < 0 || a->sp.row < 0)
        return LA_ERR_STRIDE;
    {
        const int64_t st[3] = {a->sp.row, a->sp.head, a->sp.slot};
        const int64_t ex[3] = {a->V, a->HV, a->pool_size};
        if (!no_overlap(3, st, ex, a->K))
            return LA_ERR_STRIDE;
    }
    const int64_t es = a->state_dtype == LA_BF16 ? 2 : 4;
    if ((static_cast<int64_t>(a->V - 1) * a->sp.row + a->K) * es > INT32_MAX)
        return LA_ERR_STRIDE;
    const int64_t epc = 16 / es;
    if (!aligned(a->pool, 16) || (a->sp.slot % epc) || (a->sp.head % epc) ||
        (a->sp.row % epc))
        return LA_ERR_ALIGN;
    if (!aligned(a->factors, 16) || !aligned(a->read_idx, 4) ||
        !aligned(a->write_idx, 4) || !aligned(a->num_tokens, 4))
        return LA_ERR_ALIGN;

    ReplayParams p;
    p.B = a->B;
    p.T = a->T;
    p.HV = a->HV;
    p.xcd_block = xcd_block_for(a->B, a->HV);  // as the decode kernels
    p.factors = a->factors;
    p.pool = a->pool;
    p.sp_slot = a->sp.slot;
    p.sp_head = a->sp.head;
    p.sp_row = a->sp.row;
    p.ridx = a->read_idx;
    p.widx = a->write_idx;
    p.ntok = a->num_tokens;
    p.cu = a->cu_seqlens;
    p.total = a->cu_seqlens ? a->total_tokens : 0;
    const bool bs = a->state_dtype == LA_BF16;
    typedef void (*ReplayFn)(const ReplayParams);
    ReplayFn fn;
    if (a->K == 128)
        fn = a->V == 128 ? (bs ? replay_kernel<128, 128, true>
                               : replay_kernel<128, 128, false>)
                         : (bs ? replay_kernel<128, 64, true>
                               : replay_kernel<128, 64, false>);
    else
        fn = a->V == 128 ? (bs ? replay_kernel<64, 128, true>
                               : replay_kernel<64, 128, false>)
                         : (bs ? replay_kernel<64, 64, true>
                               : replay_kernel<64, 64, false>);
    void *kargs[] = {&p};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(fn),
        dim3(static_cast<unsigned>(a->B) * a->HV),
        dim3((a->V / kRowsPerWave) * 64), kargs, 0,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_check_indices(int32_t B, int32_t pool_size,
                           const int32_t *read_idx, const int32_t *write_idx,
                           int32_t *dev_result, void *stream)
{
    if (B < 0 || pool_size < 1)
        return LA_ERR_SHAPE;
    if (!dev_result || (B > 0 && !read_idx))
        return LA_ERR_NULL;
    if (!aligned(dev_result, 4) || !aligned(read_idx, 4) ||
        !aligned(write_idx, 4))
        return LA_ERR_ALIGN;
    void *kargs[] = {&B, &pool_size, &read_idx, &write_idx, &dev_result};
    return launch_check(reinterpret_cast<const void *>(check_indices_kernel),
                        B, kargs, dev_result, stream);
}

la_status la_check_token_slots(int32_t B, int32_t T, int32_t pool_size,
                               const int32_t *token_slots,
                               int64_t table_stride,
                               const int32_t *num_accepted,
                               int32_t *dev_result, void *stream)
{
    if (B < 0 || T < 1 || pool_size < 1)
        return LA_ERR_SHAPE;
    if (table_stride < T)
        return LA_ERR_STRIDE;
    if (!dev_result || (B > 0 && (!token_slots || !num_accepted)))
        return LA_ERR_NULL;
    if (!aligned(dev_result, 4) || !aligned(token_slots, 4) ||
        !aligned(num_accepted, 4))
        return LA_ERR_ALIGN;
    void *kargs[] = {&B, &T, &pool_size, &token_slots, &table_stride,
                     &num_accepted, &dev_result};
    return launch_check(
        reinterpret_cast<const void *>(check_token_slots_kernel), B, kargs,
        dev_result, stream);
}

la_status la_check_cu_seqlens(int32_t B, int32_t T, int32_t total_tokens,
                              const int32_t *cu_seqlens, int32_t *dev_result,
                              void *stream)
{
    if (B < 0 || T < 1 || total_tokens < 0)
        return LA_ERR_SHAPE;
    if (!dev_result || !cu_seqlens)
        return LA_ERR_NULL;
    if (!aligned(dev_result, 4) || !aligned(cu_seqlens, 4))
        return LA_ERR_ALIGN;
    void *kargs[] = {&B, &T, &total_tokens, &cu_seqlens, &dev_result};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(check_cu_seqlens_kernel), dim3(1),
        dim3(1024), kargs, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

const char *la_status_string(la_status s)
{
    switch (s) {
    case LA_OK:
        return "ok";
    case LA_ERR_NULL:
        return "a required pointer is NULL";
    case LA_ERR_SHAPE:
        return "a size is out of range or inconsistent";
    case LA_ERR_STRIDE:
        return "bad stride: negative, innermost != 1, or overlapping tiles";
    case LA_ERR_ALIGN:
        return "misaligned pointer or stride";
    case LA_ERR_DTYPE:
        return "unknown dtype";
    case LA_ERR_ARG:
        return "argument inconsistent with the entry point";
    case LA_ERR_UNSUPPORTED:
        return "unsupported size (K and V must be 64 or 128)";
    case LA_ERR_LAUNCH:
        return "HIP launch failed";
    }
    return "unknown status";
}

int32_t la_version(void) { return 230; }

}  // extern "C"
