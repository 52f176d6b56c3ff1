// bf16 gather-GEMM on the CDNA4 matrix cores with the weight operand
// streamed from memory straight into registers ("SV-TAD: Native Sparse
// Convolutions for Efficient Temporal Action Detection", Key Design 2: the
// wide-channel path, y_k = sum_j W_j x[N[k, j]] as an implicit GEMM with
// M = tokens, K = taps * C, N = output channels; -1 entries are zero
// padding).  Taps: 9 (3 x 3), 25 and 49 (5 x 5, 7 x 7) and 1 (1 x 1).
//
// Same product as k_conv_mfma (conv_mfma.hip),
//     out[k][c] = sum_j sum_i A[N[k, j]][i] * B[P - j][c][i]  (+ bias[c]),
// for both passes (forward: A = X; input gradient: A = dY and the mirrored
// tap), summed in the same order: 64-channel chunks, taps inside a chunk,
// four k-steps of v_mfma_f32_32x32x16_bf16 inside a tap, with the same
// operand pairing.  The two kernels therefore give bit-identical outputs and
// the dispatcher may pick either.
//
// What differs is where the operands live and how the chip is filled.
//   - The weights are repacked once per call into fragment order (below): a
//     B fragment (one k-step, 32 output channels) is one contiguous
//     kilobyte, loaded by one fully coalesced 16-byte-per-lane buffer load
//     straight into registers, one round ahead of its use.  No weight tile
//     passes through LDS, so there is no barrier per round.
//   - Only the gathered rows (the tile's neighbour window) sit in LDS,
//     brought in by direct-to-LDS buffer loads (no staging registers) and
//     double-buffered per 64-channel chunk: one barrier per chunk.
//   - Each wave owns MB * 32 tokens x NB * 32 output channels (MB x NB
//     blocks of 32 x 32, accumulators in the AGPRs; NB = 4, or 2 where the
//     smaller tile fills more of the chip).  An MFMA then costs 256 bytes of
//     LDS reads and 256 bytes of weight loads when MB = NB = 4; k_conv_mfma's
//     64 x 64 blocks read 512 bytes of LDS per MFMA, the whole LDS bandwidth
//     of a compute unit when all four SIMDs issue.
//   - Workgroup: 4 waves, 2 x 2, tile 64 MB tokens x 64 NB channels, one
//     workgroup (one wave per SIMD) per compute unit.  The host picks the
//     smallest tile (MB in {2, 3, 4}, NB in {2, 4}) whose grid is one round
//     of at most 256 tiles where it can.  Measured on the c5 stages: with two workgroups per compute unit
//     the shader clock fell to ~1.7 GHz against ~2.1 GHz with one, and a
//     lone wave per SIMD issues MFMAs back to back (32 cycles each) when its
//     operands are in flight early enough, which the software pipelining
//     below arranges.
//
// Fragment order of B (K % 64 == 0, NO % 128 == 0), 16-byte pieces:
//   Bf[r][g][ks][nb][lane] = B(j, k, col) for e = 0..7 along k, with
//   round r = c * TAPS + j (chunk c of 64 contracted channels, tap j),
//   g = 64-channel group of the output, ks = k-step of 16, nb = 32-column
//   block, k = 64c + 16ks + 8(lane >> 5) + e, col = 64g + 32nb + (lane & 31),
//   and B(j, k, col) = Wt[j][k][col] for the forward (K = C_in, NO = C_out)
//   or Wt[TAPS - 1 - j][col][k] for the input gradient (K = C_out,
//   NO = C_in).
//
// Window rows are 128 bytes (64 channels) without padding; the 16-byte piece
// p of row r sits at slot p ^ ((r >> 1) & 7).  A fragment read of 16 rows
// by 16 lanes covers the 64 LDS banks once when the rows are consecutive
// (row parity picks the 128-byte half, the swizzle the slot).
#include "internal.h"
#include "mfma.h"

namespace svc {

constexpr int BF_WAVES = 4;              // waves per workgroup (2 x 2)
constexpr int BF_KC = 64;                // contracted channels per chunk
constexpr int BF_HALO = 32;              // window rows on either side of the tile
constexpr int BF_ROWB = 128;             // bytes per window row
constexpr int BF_MAXTILES = 256;         // one workgroup per compute unit of a 256-CU part

typedef __attribute__((address_space(3))) void lds_void_t;

// The second problem of a paired launch: same N, taps and tile shape, no
// bias; its tiles follow the first problem's `tiles1`.
struct BfragSecond {
    const uint16_t* A;
    const uint16_t* Bf;
    uint16_t* out;
    int K, NO, tiles1;
};

// MB: 32-row blocks of tokens per wave, NB: 32-column blocks of output
// channels per wave; tile 64 * MB tokens x 64 * NB channels.  PAIR: the
// grid also holds the tiles of a second problem on the same N (the chunk
// driver's forward and input gradient), so that two problems too small to
// fill the chip run side by side in one launch.
template <int TAPS, int MB, int NB, bool PAIR>
__global__ __launch_bounds__(64 * BF_WAVES, 1) void k_conv_bfrag(const uint16_t* __restrict__ A1,
                                                               const int32_t* __restrict__ Nt,
                                                               const uint16_t* __restrict__ B1,
                                                               const uint16_t* __restrict__ bias1,
                                                               uint16_t* __restrict__ out1, int n, int K1, int NO1,
                                                               BfragSecond p2) {
    constexpr int BM = 64 * MB, BN = 64 * NB, NT = 64 * BF_WAVES;
    int logical = xcd_remap(blockIdx.x, gridDim.x);
    bool second = false;
    if constexpr (PAIR) second = logical >= p2.tiles1;
    if (second) logical -= p2.tiles1;
    const uint16_t* __restrict__ A = second ? p2.A : A1;
    const uint16_t* __restrict__ Bf = second ? p2.Bf : B1;
    const uint16_t* __restrict__ bias = second ? nullptr : bias1;
    uint16_t* __restrict__ out = second ? p2.out : out1;
    const int K = second ? p2.K : K1, NO = second ? p2.NO : NO1;
    static_assert(NB == 2 || NB == 4, "a wave's channels are whole 64-channel groups");
    // Window rows are requested before the tile's N slice has arrived, from
    // the fixed start k0 - HALO: with tokens packed frame-major and in
    // ascending flat order inside a frame, every neighbour of token k at
    // most R rows and columns away (K = 2R + 1) lies within R (W + 1) packed
    // positions of k.  So the tile's rows fall inside [k0 - HALO,
    // k0 + BM + HALO) with HALO = 32 for 3 x 3 on grids up to 31 wide, and
    // HALO = 64 for 5 x 5 (up to 31 wide) and 7 x 7 (up to 20 wide).  Tiles
    // whose rows do not (other packings, wider grids) switch to gather mode.
    // With one tap (1 x 1) the rows are the tile's own: no halo.
    constexpr int HALO = TAPS == 1 ? 0 : (TAPS == 9 ? BF_HALO : 2 * BF_HALO);
    constexpr int WIN = BM + 2 * HALO;
    constexpr int ZROW = WIN;                       // all-zero row: target of -1 entries
    constexpr int WB = (WIN + 1) * BF_ROWB;         // bytes per window buffer
    // Two buffers as two arrays, used through compile-time choices only: the
    // compiler then sees that the direct loads into one never alias the
    // fragment reads from the other, and waits for them only at a barrier.
    __shared__ __align__(16) char sW0[WB];
    __shared__ __align__(16) char sW1[WB];
    __shared__ int sN[BM * TAPS];
    __shared__ int sOut;                            // some entry lies outside the window

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;        // token half, channel half of the tile
    const int l32 = lane & 31, lhi = lane >> 5;
    const int tilesN = NO / BN;
    const int k0 = (logical / tilesN) * BM;
    const int n0 = (logical % tilesN) * BN;
    const int nchunks = K / BF_KC;
    const int R = nchunks * TAPS;
    const int wlo = max(0, k0 - HALO);

    const rsrc_t rA = make_rsrc(A, static_cast<uint32_t>(n) * K * 2);
    const rsrc_t rB = make_rsrc(Bf, static_cast<uint32_t>(TAPS) * NO * K * 2);
    const rsrc_t rN = make_rsrc(Nt, static_cast<uint32_t>(n) * TAPS * 4);
    // Direct loads: lane L of an instruction writes 16 bytes at the
    // instruction's LDS base + 16 L, i.e. row L >> 3, slot L & 7 of the
    // instruction's 8 rows; it fetches the piece that belongs in that slot.
    const int drow = lane >> 3, dslot = lane & 7;
    // Window of chunk c: rows wlo .. wlo + WIN - 1 (rows past n read as
    // zeros through the range check).
    auto stage_window = [&](int c, char* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < WIN / 8 / BF_WAVES; ++u) {
            const int b = wave + BF_WAVES * u;
            const int row = b * 8 + drow;
            const int gp = dslot ^ ((row >> 1) & 7);
            const uint32_t off = (static_cast<uint32_t>(wlo + row) * K + c * BF_KC + gp * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t*)(buf + b * 1024), 16,
                                                     wlo + row < n ? off : kOob, 0, 0, 0);
        }
    };
    // Gather mode: the tile's rows through tap j of round rr, row i of the
    // tile at window row i (-1 entries read as zeros).
    auto stage_gather = [&](int rr, char* buf) __attribute__((always_inline)) {
        const int c = rr / TAPS, j = rr - c * TAPS;
#pragma unroll
        for (int u = 0; u < BM / 8 / BF_WAVES; ++u) {
            const int b = wave + BF_WAVES * u;
            const int row = b * 8 + drow;
            const int mm = sN[row * TAPS + j];
            const int gp = dslot ^ ((row >> 1) & 7);
            const uint32_t off = mm >= 0 ? (static_cast<uint32_t>(mm) * K + c * BF_KC + gp * 8) * 2 : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t*)(buf + b * 1024), 16, off, 0, 0, 0);
        }
    };
    // B fragments of round rr for this wave's NB * 32 output channels (NB / 2
    // 64-channel groups): a per-lane offset in one register and a uniform one
    // in a scalar register.  The loads issued during the last round re-read
    // that round (unused).
    const uint32_t bLane = static_cast<uint32_t>(lane * 16);
    const uint32_t bWave = static_cast<uint32_t>((n0 / 64 + (NB / 2) * wn) * 8192);
    const uint32_t bRound = static_cast<uint32_t>(NO / 64) * 8192;
    auto loadB = [&](int rr, int ks, int nb) __attribute__((always_inline)) {     // nb < NB: 32-column block of the wave
        const uint32_t so = bWave + static_cast<uint32_t>(min(rr, R - 1)) * bRound + (nb >> 1) * 8192 +
                            (ks * 2 + (nb & 1)) * 1024;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rB, bLane, __builtin_amdgcn_readfirstlane(so), 0);
        return __builtin_bit_cast(bf16x8_t, v);
    };

    floatx16_t acc[MB][NB];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = zero16();
    bf16x8_t bq[4][NB];

    // ---- prologue: the N slice, the speculative window of chunk 0 and the
    // first round's B fragments are all requested before anything waits.
    constexpr int NE = (BM * TAPS + NT - 1) / NT;
    int m[NE];
    {
        const uint32_t base = static_cast<uint32_t>(k0) * TAPS * 4;
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = tid + NT * u;
            m[u] = load4(rN, e < BM * TAPS ? base + e * 4 : kOob);    // rows past n read as 0
        }
    }
    if (tid == 0) sOut = 0;
    if (tid < 16)
        *reinterpret_cast<uint4*>((tid < 8 ? sW0 : sW1) + ZROW * BF_ROWB + (tid & 7) * 16) = make_uint4(0, 0, 0, 0);
    stage_window(0, sW0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bq[ks][nb] = loadB(0, ks, nb);
    __syncthreads();                     // sOut cleared
    {
        bool outside = false;
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = tid + NT * u;
            const bool row_ok = e < BM * TAPS && k0 + e / TAPS < n;
            const int v = row_ok ? clamp_index(m[u], n) : -1;
            if (e < BM * TAPS) sN[e] = v;
            outside |= v >= 0 && (v < wlo || v >= wlo + WIN);
        }
        if (__builtin_amdgcn_ballot_w64(outside) != 0 && lane == 0) sOut = 1;
    }
    __syncthreads();                     // also waits for the direct loads
    const bool window = sOut == 0;

    // Rows of tap j: byte offset of the window row of each of this lane's
    // MB tokens (the tile row in gather mode; -1 entries to the zero row).
    const int tok0 = wm * MB * 32 + l32;
    auto entries = [&](int j, int* mm) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) mm[mb] = sN[(tok0 + mb * 32) * TAPS + j];
    };
    auto rows_from = [&](const int* mm, bool win, int* rowb) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            rowb[mb] = (mm[mb] < 0 ? ZROW : (win ? mm[mb] - wlo : tok0 + mb * 32)) * BF_ROWB;
    };
    auto read_a = [&](const char* buf, const int* rowb, int ks, bf16x8_t* a) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int sw = (rowb[mb] >> 8) & 7;      // (row >> 1) & 7
            a[mb] = frag_row(reinterpret_cast<const uint16_t*>(buf + rowb[mb] + (((2 * ks + lhi) ^ sw) << 4)));
        }
    };
    // The rounds of one buffer (taps j0 .. j1 - 1 of chunk c, or one tap in
    // gather mode).  Each k-step's MFMAs use A fragments read one k-step
    // earlier; the next tap's N entries are read during the first k-step,
    // turned into rows during the second and its first fragments read
    // during the last; each k-step's B registers take the next round's
    // fragments right after its MFMAs.  Scheduling barriers keep that
    // order: left to itself the compiler issued the reads after the MFMAs
    // they were meant to overlap, and sank the B loads to the end of the
    // round.
    auto rounds = [&](const char* buf, int c, int j0, int j1, bool win) __attribute__((always_inline)) {
        int rowb[MB], rown[MB], mn[MB];
        bf16x8_t a[MB], an[MB];
        entries(j0, mn);
        rows_from(mn, win, rowb);
        read_a(buf, rowb, 0, a);
        for (int j = j0; j < j1; ++j) {
            const int rr = c * TAPS + j;
            const bool more = j + 1 < j1;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks == 0 && more) entries(j + 1, mn);
                if (ks == 1 && more) rows_from(mn, win, rown);
                if (ks < 3) read_a(buf, rowb, ks + 1, an);
                else if (more) read_a(buf, rown, 0, an);
                // MFMAs column block by column block, so that B register
                // nb is free for the next round's fragment after MB MFMAs.
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma32(a[mb], bq[ks][nb], acc[mb][nb]);
                    bq[ks][nb] = loadB(rr + 1, ks, nb);
                }
                // Issue order: one A read after each of the first MFMAs,
                // each B load right after the last MFMA that reads its
                // register.  A wave issues in order, so loads and reads
                // queued behind the k-step's MFMAs would wait for their
                // issue; between them they go out in the MFMAs' shadow.
                if (ks < 3 || more) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x008, MB, 0);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (nb > 0) __builtin_amdgcn_sched_group_barrier(0x008, MB, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) a[mb] = an[mb];
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) rowb[mb] = rown[mb];
        }
    };

    if (window) {
        // Chunk c reads buffer c & 1 while chunk c + 1's window loads into
        // the other one (last read in chunk c - 1, before the barrier that
        // ended it); one barrier per chunk.
        auto chunk = [&](int c, const char* cur, char* nxt) __attribute__((always_inline)) {
            if (c + 1 < nchunks) stage_window(c + 1, nxt);
            rounds(cur, c, 0, TAPS, true);
            if (c + 1 < nchunks) __syncthreads();
        };
        int c = 0;
        for (; c + 1 < nchunks; c += 2) {
            chunk(c, sW0, sW1);
            chunk(c + 1, sW1, sW0);
        }
        if (c < nchunks) chunk(c, sW0, sW1);
    } else {
        // Gather mode: round rr's rows sit in buffer rr & 1; round rr + 1's
        // load into the other one; one barrier per round.  (The speculative
        // window in sW0 landed before the barrier above.)
        stage_gather(0, sW0);
        __syncthreads();
        auto ground = [&](int rr, const char* cur, char* nxt) __attribute__((always_inline)) {
            if (rr + 1 < R) stage_gather(rr + 1, nxt);
            const int c = rr / TAPS, j = rr - c * TAPS;
            rounds(cur, c, j, j + 1, false);
            __syncthreads();
        };
        int rr = 0;
        for (; rr + 1 < R; rr += 2) {
            ground(rr, sW0, sW1);
            ground(rr + 1, sW1, sW0);
        }
        if (rr < R) ground(rr, sW0, sW1);
    }

    // ---- epilogue: bias, round to bf16 and store straight from the
    // accumulators.  Lane l holds column l & 31 of rows 8g + 4(l >> 5) + q of
    // each 32 x 32 block, so a store instruction writes two 64-byte row
    // pieces; rows past n get an out-of-range offset.  Staging the tile in
    // LDS for 16-byte stores cost more: the 2-byte LDS writes of four waves
    // and the barriers between passes took about a tenth of the kernel.
    const rsrc_t rO = make_rsrc(out, static_cast<uint32_t>(n) * NO * 2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = n0 + wn * (NB * 32) + nb * 32 + l32;
        const float bv = bias ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int orow = k0 + wm * MB * 32 + mb * 32 + g * 8 + lhi * 4 + q;
                    const uint32_t off = orow < n ? (static_cast<uint32_t>(orow) * NO + col) * 2 : kOob;
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[mb][nb][g * 4 + q] + bv), rO, off, 0, 0);
                }
    }
}

// Repack into fragment order (see the top of this file); one thread per
// 16-byte piece, written in order.
template <bool DX>
__global__ __launch_bounds__(256) void k_repack_frag(const uint16_t* __restrict__ Wt, uint16_t* __restrict__ Bf,
                                                     int taps, int Ci, int Co) {
    const int K = DX ? Co : Ci, NO = DX ? Ci : Co;
    const int NG = NO / 64;
    const int64_t total = static_cast<int64_t>(taps) * K * NO / 8;
    for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
         idx += static_cast<int64_t>(gridDim.x) * 256) {
        const int lane = static_cast<int>(idx & 63);
        int64_t t = idx >> 6;
        const int nb = static_cast<int>(t & 1);
        t >>= 1;
        const int ks = static_cast<int>(t & 3);
        t >>= 2;
        const int g = static_cast<int>(t % NG);
        const int64_t rr = t / NG;
        const int c = static_cast<int>(rr / taps), j = static_cast<int>(rr % taps);
        const int k = 64 * c + 16 * ks + 8 * (lane >> 5);
        const int col = 64 * g + 32 * nb + (lane & 31);
        uint4 v;
        if (DX) {
            v = *reinterpret_cast<const uint4*>(Wt + (static_cast<int64_t>(taps - 1 - j) * Ci + col) * Co + k);
        } else {
            uint32_t w[4];
            const uint16_t* s = Wt + (static_cast<int64_t>(j) * Ci + k) * Co + col;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                w[p] = static_cast<uint32_t>(s[(2 * p) * Co]) | (static_cast<uint32_t>(s[(2 * p + 1) * Co]) << 16);
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *reinterpret_cast<uint4*>(Bf + idx * 8) = v;
    }
}

// Several layers' weights in one launch: blockIdx.y = (layer, layout), the
// layout's fragment order as k_repack_frag writes it.
struct RepackBatch {
    const uint16_t* W[kRepackMax];
    uint16_t* out[2][kRepackMax];     // [0]: forward (nullable), [1]: input gradient (nullable)
};

__global__ __launch_bounds__(256) void k_repack_batch(RepackBatch b, int taps, int Ci, int Co) {
    const int layer = blockIdx.y >> 1, dx = blockIdx.y & 1;
    uint16_t* Bf = b.out[dx][layer];
    if (!Bf) return;
    const uint16_t* Wt = b.W[layer];
    const int K = dx ? Co : Ci, NO = dx ? Ci : Co;
    const int NG = NO / 64;
    const int64_t total = static_cast<int64_t>(taps) * K * NO / 8;
    for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
         idx += static_cast<int64_t>(gridDim.x) * 256) {
        const int lane = static_cast<int>(idx & 63);
        int64_t t = idx >> 6;
        const int nb = static_cast<int>(t & 1);
        t >>= 1;
        const int ks = static_cast<int>(t & 3);
        t >>= 2;
        const int g = static_cast<int>(t % NG);
        const int64_t rr = t / NG;
        const int c = static_cast<int>(rr / taps), j = static_cast<int>(rr % taps);
        const int k = 64 * c + 16 * ks + 8 * (lane >> 5);
        const int col = 64 * g + 32 * nb + (lane & 31);
        uint32_t w[4];
        if (dx) {
            const uint16_t* s = Wt + (static_cast<int64_t>(taps - 1 - j) * Ci + col) * Co + k;
#pragma unroll
            for (int p = 0; p < 4; ++p) w[p] = static_cast<uint32_t>(s[2 * p]) | (static_cast<uint32_t>(s[2 * p + 1]) << 16);
        } else {
            const uint16_t* s = Wt + (static_cast<int64_t>(j) * Ci + k) * Co + col;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                w[p] = static_cast<uint32_t>(s[(2 * p) * Co]) | (static_cast<uint32_t>(s[(2 * p + 1) * Co]) << 16);
        }
        *reinterpret_cast<uint4*>(Bf + idx * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_repack_batch(int count, const uint16_t* const* W, uint16_t* const* V, uint16_t* const* P, int Ci,
                               int Co, int taps, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    if (count > kRepackMax) return hipErrorInvalidValue;
    RepackBatch b{};
    for (int i = 0; i < count; ++i) {
        b.W[i] = W[i];
        b.out[0][i] = V ? V[i] : nullptr;
        b.out[1][i] = P ? P[i] : nullptr;
    }
    const int64_t total = static_cast<int64_t>(taps) * Ci * Co / 8;
    const int bx = static_cast<int>(std::min<int64_t>((total + 255) / 256, 1024));
    hipLaunchKernelGGL(k_repack_batch, dim3(bx, 2 * count), dim3(256), 0, stream, b, taps, Ci, Co);
    return hipGetLastError();
}

// 1 x 1 only with at least 8 rounds (512 contracted channels): with fewer,
// prologue and epilogue dominate and k_conv_mfma's two workgroups per CU
// overlap them better (c3a at 1 x 1: forward 14.4 against 18.9 us).
bool conv_bfrag_ok(int K, int NO, int taps) {
    return (taps == 9 || taps == 25 || taps == 49 || (taps == 1 && K >= 512)) && K > 0 && NO > 0 &&
           K % BF_KC == 0 && NO % 128 == 0 && static_cast<int64_t>(taps) * NO * K * 2 <= kMaxRange;
}

// The paired launch is built for 3 x 3 and 1 x 1 only.
bool conv_bfrag_pair_ok(int K1, int NO1, int K2, int NO2, int taps) {
    return (taps == 1 || taps == 9) && conv_bfrag_ok(K1, NO1, taps) && conv_bfrag_ok(K2, NO2, taps);
}

hipError_t launch_repack_frag(const uint16_t* Wt, uint16_t* Bf, int Ci, int Co, int taps, bool dx,
                              hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(taps) * Ci * Co / 8;
    const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 4096));
    if (dx)
        hipLaunchKernelGGL(k_repack_frag<true>, dim3(blocks), dim3(256), 0, stream, Wt, Bf, taps, Ci, Co);
    else
        hipLaunchKernelGGL(k_repack_frag<false>, dim3(blocks), dim3(256), 0, stream, Wt, Bf, taps, Ci, Co);
    return hipGetLastError();
}

// Tile shape: the smallest tile (fewest tokens x channels per workgroup)
// whose grid is one round of at most 256 tiles (one per compute unit of a
// 256-CU part); at equal size, 256 channels (NB = 4: half the A reads per
// MFMA).  Without such a tile, the largest one the channel count allows.
// A paired launch (NO2 > 0) counts both problems' tiles against `slots` and
// needs a shape that divides both channel counts.  Depends on the arguments
// only; every shape gives the same bits.
struct BfragShape {
    int mb, nb;
};
static int64_t bfrag_tiles(BfragShape t, int64_t n, int NO) {
    return NO > 0 ? ((n + 64 * t.mb - 1) / (64 * t.mb)) * (NO / (64 * t.nb)) : 0;
}
static BfragShape bfrag_shape(int64_t n, int NO, int NO2 = 0, int slots = BF_MAXTILES) {
    static const BfragShape order[] = {{2, 2}, {3, 2}, {2, 4}, {4, 2}, {3, 4}, {4, 4}};    // by tile size
    for (const BfragShape& t : order) {
        if (NO % (64 * t.nb) != 0 || NO2 % (64 * t.nb) != 0) continue;
        if (bfrag_tiles(t, n, NO) + bfrag_tiles(t, n, NO2) <= slots) return t;
    }
    return NO % 256 == 0 && NO2 % 256 == 0 ? BfragShape{4, 4} : BfragShape{4, 2};
}

template <int TAPS, bool PAIR>
static void launch_bfrag_taps(BfragShape t, dim3 grid, hipStream_t stream, const uint16_t* A, const int32_t* N,
                              const uint16_t* Bf, const uint16_t* bias, uint16_t* out, int n, int K, int NO,
                              const BfragSecond& p2) {
    const dim3 block(64 * BF_WAVES);
    if (t.nb == 2 && t.mb == 2)
        hipLaunchKernelGGL((k_conv_bfrag<TAPS, 2, 2, PAIR>), grid, block, 0, stream, A, N, Bf, bias, out, n, K, NO, p2);
    else if (t.nb == 2 && t.mb == 3)
        hipLaunchKernelGGL((k_conv_bfrag<TAPS, 3, 2, PAIR>), grid, block, 0, stream, A, N, Bf, bias, out, n, K, NO, p2);
    else if (t.nb == 2)
        hipLaunchKernelGGL((k_conv_bfrag<TAPS, 4, 2, PAIR>), grid, block, 0, stream, A, N, Bf, bias, out, n, K, NO, p2);
    else if (t.mb == 2)
        hipLaunchKernelGGL((k_conv_bfrag<TAPS, 2, 4, PAIR>), grid, block, 0, stream, A, N, Bf, bias, out, n, K, NO, p2);
    else if (t.mb == 3)
        hipLaunchKernelGGL((k_conv_bfrag<TAPS, 3, 4, PAIR>), grid, block, 0, stream, A, N, Bf, bias, out, n, K, NO, p2);
    else
        hipLaunchKernelGGL((k_conv_bfrag<TAPS, 4, 4, PAIR>), grid, block, 0, stream, A, N, Bf, bias, out, n, K, NO, p2);
}

hipError_t launch_conv_bfrag(const uint16_t* A, const int32_t* N, const uint16_t* Bf, const uint16_t* bias,
                             uint16_t* out, int64_t n, int K, int NO, int taps, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    if (!conv_bfrag_ok(K, NO, taps)) return hipErrorInvalidValue;
    const BfragShape t = bfrag_shape(n, NO);
    const dim3 grid(static_cast<unsigned>(bfrag_tiles(t, n, NO)));
    const int ni = static_cast<int>(n);
    const BfragSecond none{};
    switch (taps) {
        case 1: launch_bfrag_taps<1, false>(t, grid, stream, A, N, Bf, bias, out, ni, K, NO, none); break;
        case 9: launch_bfrag_taps<9, false>(t, grid, stream, A, N, Bf, bias, out, ni, K, NO, none); break;
        case 25: launch_bfrag_taps<25, false>(t, grid, stream, A, N, Bf, bias, out, ni, K, NO, none); break;
        default: launch_bfrag_taps<49, false>(t, grid, stream, A, N, Bf, bias, out, ni, K, NO, none); break;
    }
    return hipGetLastError();
}

hipError_t launch_conv_bfrag_pair(const uint16_t* A1, const uint16_t* B1, const uint16_t* bias1, uint16_t* out1,
                                  int K1, int NO1, const uint16_t* A2, const uint16_t* B2, uint16_t* out2, int K2,
                                  int NO2, const int32_t* N, int64_t n, int taps, int slots, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    if (!conv_bfrag_pair_ok(K1, NO1, K2, NO2, taps) || slots < 1) return hipErrorInvalidValue;
    const BfragShape t = bfrag_shape(n, NO1, NO2, slots);
    const int64_t tiles1 = bfrag_tiles(t, n, NO1);
    const dim3 grid(static_cast<unsigned>(tiles1 + bfrag_tiles(t, n, NO2)));
    const int ni = static_cast<int>(n);
    const BfragSecond p2{A2, B2, out2, K2, NO2, static_cast<int>(tiles1)};
    if (taps == 1)
        launch_bfrag_taps<1, true>(t, grid, stream, A1, N, B1, bias1, out1, ni, K1, NO1, p2);
    else
        launch_bfrag_taps<9, true>(t, grid, stream, A1, N, B1, bias1, out1, ni, K1, NO1, p2);
    return hipGetLastError();
}

}  // namespace svc
