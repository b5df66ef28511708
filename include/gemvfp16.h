/*
 * gemvfp16 -- fp16 NT matrix product, split-K matrix product and GEMV for
 * AMD Instinct MI355X (gfx950), as a C-ABI shared library (libgemvfp16.so).
 *
 * Common conventions for every entry point
 *  - fp16 means IEEE binary16; fp16 buffers are passed as void* and hold raw
 *    binary16 bit patterns.  Every matrix is row-major and contiguous.
 *  - Every data pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *    tensor).  The caller allocates and owns every buffer; the library keeps
 *    no pointer after the call returns and allocates nothing the caller sees.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on that stream and never synchronise; buffers
 *    must stay alive until that work has completed.
 *  - Outputs are overwritten (no alpha/beta) and must not alias any input.
 *  - Return value: GF_OK, or a GF_ERR_* code (gf_status_string() names it).
 *    Argument errors are detected on the host before anything is enqueued.
 *    A fault that happens later on the device surfaces at the caller's next
 *    synchronisation, as with any HIP library.  Nothing is printed.
 *  - Degenerate shapes: M == 0 or N == 0 is a no-op returning GF_OK; K == 0
 *    writes +0 everywhere (the empty sum).
 *  - Any M, N, K >= 0 is accepted.  The fast path (128-bit loads and stores)
 *    is taken when every base pointer is 16-byte aligned and K % 8 == 0
 *    (and N % 8 == 0 for the fp16 C stores); otherwise a masked path that
 *    needs only 2-byte alignment computes the same result.
 *  - Each operand must be smaller than 2^31 elements.
 */
#ifndef GEMVFP16_H
#define GEMVFP16_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GF_OK = 0,
    GF_ERR_INVALID_ARG = 1,   /* bad size, NULL or misaligned pointer, bad mode */
    GF_ERR_HIP = 2,           /* the HIP runtime reported an error at launch */
    GF_ERR_UNSUPPORTED = 3,   /* no compiled kernel for the requested config */
    GF_ERR_TOO_LARGE = 4      /* the problem exceeds the library's fixed scratch (no-allocation call) */
};

enum { GF_SPLITK_ATOMIC = 0, GF_SPLITK_TWOPASS = 1, GF_SPLITK_F16 = 2 };

/*
 * C = A . B^T.  A is M x K fp16, B is N x K fp16, C is M x N fp16.
 * Products are accumulated in fp32 and each result is rounded once to fp16
 * (round-to-nearest-even).
 * Defined by the TileLang FP16 matmul autotune benchmark page, sections 1
 * and 2 (C = A B^T with A(M,K), B(N,K), C(M,N), fp16 operands, fp32
 * accumulation, transpose_B) and the autotune tutorial page's reference().
 * The library picks the launch: M <= 16 takes the skinny kernel, and so do
 * 17 <= M <= 64 when N <= 8192, K >= 4096 and K % 512 == 0; when the
 * default tile would leave its last round of workgroups at most half full,
 * the call enqueues two launches on `stream`, the leading rows of C in whole
 * rounds and the rest with a smaller tile (same result bits as one launch
 * of the default tile, except where the rest is 16 rows or fewer and takes
 * the skinny kernel).
 */
int gemm_f16_nt(const void* A, const void* B, void* C, int M, int N, int K, void* stream);

/*
 * Split-K form of the same product with an fp32 output:
 * C32 = A . B^T, A M x K fp16, B N x K fp16, C32 M x N float.
 * K is cut into split_k contiguous slices (tile-aligned; the last may be
 * short and any may be empty); each slice's partial product is computed by
 * its own workgroups and added into C32 with fp32 global atomics.  C32 is
 * zeroed by the call itself, on the stream.  The order of the atomic adds is
 * not fixed, so results can differ in the last bits from run to run (they
 * are exact whenever every partial sum is exactly representable).
 * split_k must be >= 1.
 * Defined by the "basic GEMM to SplitK" page, SplitK section (grid dimension
 * over K slices, out_dtype float32, per-element atomic add into C).
 */
int gemm_f16_nt_splitk(const void* A, const void* B, float* C32, int M, int N, int K,
                       int split_k, void* stream);

/*
 * y = W . x.  W is N x K fp16, x has K fp16 entries, y has N fp16 entries.
 * fp32 accumulation, one rounding to fp16 (round-to-nearest-even).
 * Defined by the TileLang GEMV page: GEMV as the degenerate (1,k) x (k,n)
 * GEMM, kernels with A(K,), B(N,K), C(N,) accumulated in float (here x = A,
 * W = B, y = C).
 */
int gemv_f16(const void* W, const void* x, void* y, int N, int K, void* stream);

/* ---- extensions ------------------------------------------------------ */

/*
 * fp16 GEMM with other operand layouts: C = op(A) . op(B) with C M x N fp16,
 * fp32 accumulation and one rounding to fp16 (round-to-nearest-even), as
 * for gemm_f16_nt.
 *   a_kmajor = 0: A is M x K (K contiguous);  1: A is K x M (M contiguous).
 *   b_kmajor = 0: B is N x K (K contiguous);  1: B is K x N (N contiguous).
 * (0, 0) is gemm_f16_nt.  gemm_f16_nn = (0, 1): C = A . B with B K x N, the
 * plain row-major product.  gemm_f16_tn = (1, 1): C = A^T . B.  The fast path
 * needs 16-byte aligned A, B, C and a multiple of 8 for each operand's
 * contiguous extent; anything else runs a masked path with the same result.
 * Returns GF_ERR_INVALID_ARG for a flag other than 0 or 1.
 * Defined by the "basic GEMM to SplitK" page, basic GEMM section (the
 * row-major product of an M x K and a K x N matrix, C[i][j] the sum over k
 * of A[i][k] B[k][j]); the TileLang FP16 matmul page, section 2, names the
 * B^T operand form of gemm_f16_nt.
 */
int gemm_f16(const void* A, const void* B, void* C, int M, int N, int K, int a_kmajor, int b_kmajor,
             void* stream);
int gemm_f16_nn(const void* A, const void* B, void* C, int M, int N, int K, void* stream);
int gemm_f16_tn(const void* A, const void* B, void* C, int M, int N, int K, void* stream);

/* Bytes of workspace gemm_f16_nt_splitk_ex needs in GF_SPLITK_TWOPASS mode:
 * split_k * M * N * sizeof(float) (0 for invalid arguments). */
size_t gemm_f16_nt_splitk_workspace_bytes(int M, int N, int split_k);

/*
 * Split-K with a choice of combine.  mode = GF_SPLITK_ATOMIC behaves exactly
 * like gemm_f16_nt_splitk (workspace ignored, may be NULL).
 * mode = GF_SPLITK_TWOPASS: pass 1 stores slice s's partial tile into
 * workspace[s][M][N] (fp32, caller-owned device memory of at least
 * gemm_f16_nt_splitk_workspace_bytes(M, N, split_k) bytes, at least 4-byte
 * aligned; with 16-byte alignment and M*N % 4 == 0 the reduce uses float4);
 * pass 2 sums the slices in ascending s into C32.  The two-pass result is
 * bitwise reproducible from run to run.
 * Returns GF_ERR_INVALID_ARG for a bad mode or a NULL / short workspace in
 * two-pass mode.
 */
int gemm_f16_nt_splitk_ex(const void* A, const void* B, float* C32, int M, int N, int K,
                          int split_k, int mode, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Two-pass split-K (GF_SPLITK_TWOPASS semantics: fp32 C32 = A . B^T, the
 * slices summed in ascending order, bitwise reproducible, the same bits as
 * gemm_f16_nt_splitk_ex in that mode) that allocates nothing and takes no
 * workspace: for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The slice partials go to a scratch array that the library holds in device
 * memory, gf_noalloc_scratch_bytes() = 64 MiB on each GPU it runs on, until
 * the process ends.  The caller still passes A, B and C32.
 * Limit: split_k * M * N * 4 bytes must fit the scratch (GF_ERR_TOO_LARGE
 * otherwise, checked on the host before anything is enqueued; 1024 x 1024
 * fits split_k <= 16).  Every call on one GPU shares that GPU's scratch: two
 * calls that overlap on one GPU (on different streams or host threads) race
 * and must be serialised by the caller.  The scratch used is that of the
 * device `stream` belongs to (the current device for the null stream); the
 * first call on a device looks up its address there (hipGetSymbolAddress,
 * with that device made current for the lookup and the caller's device
 * restored; GF_ERR_HIP if that fails).  Other errors as
 * gemm_f16_nt_splitk_ex.
 */
int gemm_f16_nt_splitk_noalloc(const void* A, const void* B, float* C32, int M, int N, int K,
                               int split_k, void* stream);

/* Bytes of the no-allocation scratch of gemm_f16_nt_splitk_noalloc (64 MiB). */
size_t gf_noalloc_scratch_bytes(void);

/*
 * Split-K with an fp16 output: C = A . B^T, A M x K fp16, B N x K fp16,
 * C M x N fp16.  Pass 1 stores slice s's fp32 partial tile into
 * workspace[s][M][N]; pass 2 sums the slices in ascending s in fp32 and
 * rounds each sum once to fp16 (round-to-nearest-even).  The result is
 * therefore exactly the GF_SPLITK_TWOPASS fp32 result rounded to fp16, and
 * bitwise reproducible from run to run.  workspace: caller-owned device
 * memory of at least gemm_f16_nt_splitk_workspace_bytes(M, N, split_k)
 * bytes, at least 4-byte aligned (16-byte alignment of workspace and C with
 * M*N % 8 == 0 selects the vector reduce).  K == 0 writes +0 everywhere.
 * Returns GF_ERR_INVALID_ARG for split_k < 1 or a NULL / short workspace.
 * Defined by the "basic GEMM to SplitK" page, SplitK section: the split-K
 * kernel takes its output type as a parameter (there float32); this is the
 * same kernel with the fp16 output type, the fp32 slice sums rounded at the
 * end as in the TileLang FP16 matmul page's fp32-accumulate / fp16-store
 * GEMM (section 1).
 */
int gemm_f16_nt_splitk_f16(const void* A, const void* B, void* C, int M, int N, int K,
                           int split_k, void* workspace, size_t workspace_bytes, void* stream);

/* Tile configuration of the GEMM kernel (used by the offline sweep).
 * block_m x block_n x block_k tile, `stages` LDS buffers (1..4), `threads`
 * per workgroup (256 or 512).  raster: 0 = plain row-major tile order;
 * 1 = XCD-aware grouped order with panels of 10 tile-rows; n >= 2 = the
 * same with panels of n tile-rows.  schedule: 0 = every wave interleaves
 * its operand loads with its MFMAs; 1 = two wave groups alternate a memory
 * phase and an MFMA-only phase ("ping-pong", 512 threads only); 2 = one
 * wave per SIMD (256 threads), the tile barrier before the last MFMA step
 * and the next tile's first reads and loads under it; 3 = schedule 2 with
 * 16x16x32 MFMAs. */
typedef struct gf_gemm_cfg {
    int block_m, block_n, block_k, stages, threads, raster, schedule;
} gf_gemm_cfg;

/* GEMV launch shape: rows per wave, 16-byte W loads in flight per row and
 * lane, waves per workgroup, and blocks:
 *   0     = one row group per wave, the grid covers N;
 *   b > 0 = at most b workgroups that walk the row groups grid-stride.  When
 *           the fast path applies, K <= 32768 and (K/8) is a multiple of
 *           waves*64*unroll, a workgroup owns rows_per_wave rows at a time
 *           and its waves split K (partials summed through LDS); otherwise,
 *           with K <= 32768 and the fast path, each wave owns its rows and x
 *           is staged in LDS once per workgroup; otherwise as for 0.
 * Every shape gives the same result up to fp32 summation order. */
typedef struct gf_gemv_cfg {
    int rows_per_wave, unroll, waves, blocks;
} gf_gemv_cfg;

/* gemm_f16_nt with an explicit tile config; GF_ERR_UNSUPPORTED when the
 * library holds no kernel for it.  Same semantics as gemm_f16_nt. */
int gemm_f16_nt_cfg(const void* A, const void* B, void* C, int M, int N, int K,
                    const gf_gemm_cfg* cfg, void* stream);

/* Split-K with an explicit tile config (used by the offline sweep): mode
 * GF_SPLITK_ATOMIC or GF_SPLITK_TWOPASS as gemm_f16_nt_splitk_ex (C is then
 * float*), or GF_SPLITK_F16 as gemm_f16_nt_splitk_f16 (C is fp16).  Only
 * configs compiled with the fp32 epilogues qualify; GF_ERR_UNSUPPORTED
 * otherwise. */
int gemm_f16_nt_splitk_cfg(const void* A, const void* B, void* C, int M, int N, int K, int split_k,
                           int mode, void* workspace, size_t workspace_bytes, const gf_gemm_cfg* cfg,
                           void* stream);

/* gemm_f16 with an explicit tile config.  Layouts other than (0, 0) exist
 * for the configs with schedule 2, block_k 64 and block_m, block_n multiples
 * of 128; GF_ERR_UNSUPPORTED otherwise. */
int gemm_f16_cfg(const void* A, const void* B, void* C, int M, int N, int K, int a_kmajor,
                 int b_kmajor, const gf_gemm_cfg* cfg, void* stream);

/*
 * Skinny fp16 NT GEMM: gemm_f16_nt for 1 <= M <= 64 rows of A (a decode
 * batch against one large B): every byte of B is streamed once and the rows
 * of A ride along in the MFMA operand.  Same result contract as
 * gemm_f16_nt (fp32 accumulation, one fp16 rounding).  Needs A and B
 * 16-byte aligned and K % 8 == 0; 17 <= M <= 64 needs the LDS-staged form
 * (K % 512 == 0) with a ring that holds those rows: 16 * blocks + M rounded
 * up to 32, 48 or 64 rows of 1 KiB per stage, within 160 KiB and a multiple
 * of waves.  gemm_f16_nt takes this path by itself as described there; this
 * entry point runs it explicitly and returns GF_ERR_UNSUPPORTED outside
 * those conditions.  cfg: launch shape, NULL =
 * the library's choice.  waves = waves per workgroup; then one of three forms:
 *  - stages = 0, direct form on the matrix cores: blocks = 16-row blocks of
 *    B per workgroup, waves split K, loads straight to registers (unroll =
 *    k-steps per register batch, two batches in flight per wave);
 *  - stages >= 2, LDS-staged form on the matrix cores: blocks as above,
 *    1 KiB of one row per load instruction through a ring of that many
 *    512-k chunks (needs K % 512 == 0; unroll 0);
 *  - stages = 1, vector form for M <= 8: blocks = rows of B per wave, unroll
 *    = 16-byte chunks per row and lane in flight; B streamed as by gemv_f16,
 *    A staged in LDS with its rows zero-padded to whole steps of 512 * unroll
 *    k (needs M' * that padded K * 2 <= 160 KiB, M' = M rounded up to 1, 2,
 *    4 or 8; a ragged last step multiplies zeros past K);
 *  - stages = -1, split form for M <= 8: gemv_f16's split launch shape (the
 *    waves of a workgroup split K, workgroups walk whole rows of B), A held
 *    in registers; blocks = workgroups at most, unroll = 16-byte chunks per
 *    lane and row (needs K == 512 * unroll * waves).
 * Defined by the TileLang GEMV page: GEMV as the degenerate GEMM with a
 * single row of A, here with up to 16 rows (C = A B^T of the TileLang FP16
 * matmul page, section 1).
 */
typedef struct gf_skinny_cfg {
    int blocks, unroll, waves, stages;
} gf_skinny_cfg;
int gemm_f16_nt_skinny(const void* A, const void* B, void* C, int M, int N, int K,
                       const gf_skinny_cfg* cfg, void* stream);
int gf_skinny_config_count(void);
int gf_skinny_config_get(int i, gf_skinny_cfg* out);
/* The launch shape gemm_f16_nt_skinny (and gemm_f16_nt where it takes the
 * skinny kernel) would pick for a shape; GF_ERR_INVALID_ARG unless
 * 1 <= M <= 64, N >= 0, K >= 0. */
int gf_skinny_default_config(int M, int N, int K, gf_skinny_cfg* out);

/* gemv_f16 with an explicit launch shape; GF_ERR_UNSUPPORTED when the
 * library holds no kernel for it.  Same semantics as gemv_f16. */
int gemv_f16_cfg(const void* W, const void* x, void* y, int N, int K,
                 const gf_gemv_cfg* cfg, void* stream);

/* Enumerate the compiled configs: count, then the i-th (0 <= i < count).
 * The _get calls return GF_ERR_INVALID_ARG for an index out of range. */
int gf_gemm_config_count(void);
int gf_gemm_config_get(int i, gf_gemm_cfg* out);
int gf_gemv_config_count(void);
int gf_gemv_config_get(int i, gf_gemv_cfg* out);

/* The config gemm_f16_nt / gemv_f16 would pick for a shape. */
int gf_gemm_default_config(int M, int N, int K, gf_gemm_cfg* out);
int gf_gemv_default_config(int N, int K, gf_gemv_cfg* out);

/*
 * 2:4 structured sparsity of A.
 * Defined by the TileLang FP16 matmul autotune benchmark page, section 6
 * (the sparse benchmark compresses A 2:4-style into A_sparse of shape
 * (M, K/2) plus mask metadata E of shape (M, K/e_factor) and multiplies it
 * with the sparse tensor-core GEMM).  The page fixes neither which two
 * entries a group keeps nor the metadata bits; this library's format:
 *  - K must be a multiple of 16; K is cut into groups of 4 consecutive k.
 *  - A_sparse: M x K/2 fp16, row-major; group g's two kept values at 2g and
 *    2g+1, lower index first.
 *  - E: M x K/16 16-bit words, row-major; group g's field i0 | i1 << 2
 *    (i0 < i1, the kept indices within the group) sits at bits 4 * (g % 4)
 *    of word g / 4.  This is e_dtype int16 (e_factor 16); the same bytes
 *    read as int8 or int32 are the e_factor 8 and 32 forms.
 */

/*
 * Compress a dense A (M x K fp16) into A_sparse and E: each group keeps
 * its two entries of largest magnitude (compared on the fp16 bits without
 * the sign, so NaN ranks above infinity), ties going to the lower index.
 * Lossless when no group of A has more than two nonzeros.  Bit-exact,
 * deterministic.  A, A_sparse, E: device pointers, 2-byte aligned (16-byte
 * aligned A and A_sparse take the vector path).  GF_ERR_INVALID_ARG for
 * K % 16 != 0, M or K < 0, NULL or misaligned pointers, or M * K >= 2^31.
 */
int sp24_compress_f16(const void* A, void* A_sparse, void* E, int M, int K, void* stream);

/*
 * C = decompress(A_sparse, E) . B^T: the sparse product, A_sparse M x K/2
 * fp16 and E M x K/16 as above, B N x K fp16 (dense, row-major), C M x N fp16.
 * Products are accumulated in fp32 and each result is rounded once to fp16,
 * as for gemm_f16_nt.  The fast path (direct-to-LDS loads) needs A_sparse and
 * B 16-byte aligned, E 4-byte aligned and K % 32 == 0; otherwise a register-
 * staged path computes the same result.  A metadata field with i0 >= i1
 * gives an unspecified result for its row (no fault).  GF_ERR_INVALID_ARG for
 * K % 16 != 0, negative sizes, NULL or misaligned pointers, or any operand of
 * 2^31 elements or more.  M == 0 or N == 0 is a no-op; K == 0 writes +0.
 * As for gemm_f16_nt, when the default tile would leave its last round of
 * workgroups at most half full, the call enqueues two launches on `stream`
 * (the leading rows in whole rounds, the rest with a smaller tile; the same
 * result bits as one launch).
 */
int gemm_sp_f16_nt(const void* A_sparse, const void* E, const void* B, void* C, int M, int N, int K,
                   void* stream);

/* Tile config of the sparse GEMM: block_m x block_n output tile (K tiles of
 * 64), raster as in gf_gemm_cfg.  stages >= 2: that many LDS buffers, each
 * holding one K tile of A_sparse and B.  stages = 0: the paired form, which
 * loads A_sparse two K tiles and E eight K tiles at a time (fewer cache
 * lines per byte) beside two B buffers; it needs the same alignment as the
 * fast path and otherwise runs the register-staged path.  NULL = the
 * library's choice.  GF_ERR_UNSUPPORTED when no kernel is compiled for it. */
typedef struct gf_sp_cfg {
    int block_m, block_n, stages, raster;
} gf_sp_cfg;
int gemm_sp_f16_nt_cfg(const void* A_sparse, const void* E, const void* B, void* C, int M, int N, int K,
                       const gf_sp_cfg* cfg, void* stream);
int gf_sp_config_count(void);
int gf_sp_config_get(int i, gf_sp_cfg* out);
int gf_sp_default_config(int M, int N, int K, gf_sp_cfg* out);

/* Static string naming a status code. */
const char* gf_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* GEMVFP16_H */
