/*
 * gemm_preshuffle.h -- C ABI of the MI355X (gfx950) preshuffle GEMM library.
 *
 *   C[M,N] = A[M,K] . B[N,K]^T
 *
 * The problem statement is the one of the GEMM Optimization Guide (rocm
 * gemm-optimization skill), §1.1, read with §12.1 (B is N rows of K contiguous
 * elements). B is consumed in the preshuffled layout of §1.4 / §12.1; A and C
 * are plain row-major. Element types follow §6.2: INT8, FP8 (OCP E4M3FN),
 * BF16, FP16 and gfx950 MXFP4 (E2M1 values, one E8M0 scale per 32 K
 * elements), plus INT4 weights with int8 activations (W4A8, the INT4 bytes
 * formula of §8.2). The FP8 and W4A8 epilogues apply fp32 per-row /
 * per-column scales (§7.1, §8.2); every floating-point output can take the
 * fused bias / activation epilogues of the Kernel Tuning Guide, §6.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer; all data pointers are DEVICE
 *     pointers (hipMalloc'd or equivalent) unless stated otherwise. The
 *     library keeps no pointer after the call returns and allocates nothing.
 *     A plan that splits K across workgroups needs a caller-provided device
 *     workspace (gemm_ex_ws, sized by gemm_workspace_size); the other entry
 *     points never split K across workgroups and need none.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream). Nothing synchronizes; results are ready when the stream
 *     reaches that point.
 *   - Layout: A is [M][K] and C is [M][N], row-major, contiguous. Sizes are
 *     in ELEMENTS; an MXFP4 or INT4 row of K elements is K/2 bytes (element
 *     2i in the low nibble of byte i).
 *   - Shapes: N % 16 == 0 and K * (bits of a B element) % 512 == 0 (the B
 *     layout); FP8, MXFP4 and W4A8 also need K % 128 == 0 (whole MFMA K
 *     steps); M is free. When the tile does not divide M or N, the edge
 *     tiles overlap their neighbours inside M x N (no padding is needed);
 *     N below one tile or a short K runs on the small-M kernel. Which kernel
 *     and tile a call runs is the planner's choice unless gemm_opts says
 *     otherwise (gemm_plan / gemm_plan_ws report it): the small-M kernel up
 *     to 64 rows and, above, on small outputs; the tile kernel otherwise.
 *   - Thread-local state: the HIP status behind the last GP_EHIP and the
 *     runtime call that returned it (gemm_last_hip_error, gemm_last_hip_call).
 *   - Alignment: every data pointer must be 16-byte aligned.
 *   - Errors: arguments are validated on the host before any HIP call; a
 *     non-zero gp_status is returned and nothing is launched. A failing
 *     launch returns GP_EHIP. No C++ exception crosses this interface.
 *   - Thread safety: no global mutable state besides a per-device cache of
 *     the device's architecture (and the thread-local HIP status above);
 *     calls from several threads are safe.
 */
#ifndef GEMM_PRESHUFFLE_H
#define GEMM_PRESHUFFLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gp_status {
  GP_OK = 0,
  GP_EINVAL = 1,  /* null or misaligned pointer, non-positive size, bad option value */
  GP_ESHAPE = 2,  /* layout or tile divisibility violated, or size over 2^31 bytes   */
  GP_EDTYPE = 3,  /* unsupported dtype or dtype/scale combination                    */
  GP_EARCH = 4,   /* the current device is not gfx950                                */
  GP_EHIP = 5,    /* a HIP runtime call or kernel launch failed                      */
  GP_EWORKSPACE = 6 /* the plan splits K across workgroups and the call brings no
                       workspace, or one smaller than gemm_workspace_size reports    */
} gp_status;

typedef enum gp_dtype {
  GP_I8 = 0,        /* int8, two's complement                      */
  GP_FP8_E4M3 = 1,  /* OCP FP8 E4M3FN (max 448, no infinities)      */
  GP_BF16 = 2,      /* bfloat16                                     */
  GP_FP4_E2M1 = 3,  /* OCP MX FP4 E2M1, two per byte, low nibble first */
  GP_I32 = 4,       /* int32 (output of the INT8 path)              */
  GP_F16 = 5,       /* IEEE binary16                                */
  GP_I4 = 6         /* as an input type: int8 A with INT4 B (W4A8); INT4 is
                       two's complement, two per byte, low nibble first */
} gp_dtype;

/* Fused epilogue activations (Kernel Tuning Guide §6: bias, bias_relu,
 * bias_silu, bias_gelu), applied in fp32 after the scales and the bias:
 *   relu(x) = max(x, 0)   silu(x) = x / (1 + exp(-x))
 *   gelu(x) = x/2 * (1 + erf(x / sqrt 2))   (the exact, erf form)        */
typedef enum gp_act {
  GP_ACT_NONE = 0,
  GP_ACT_RELU = 1,
  GP_ACT_SILU = 2,
  GP_ACT_GELU = 3
} gp_act;

enum {
  GP_EPI_AUTO = 0,      /* planner's choice                                   */
  GP_EPI_DIRECT = 1,    /* each lane stores its accumulators (GEMM Opt. §7.1) */
  GP_EPI_CSHUFFLE = 2   /* re-map through LDS for coalesced stores (§7.2)     */
};

enum {
  GP_KERNEL_AUTO = 0,
  GP_KERNEL_TILE = 1,    /* LDS ping-pong tile kernel (GEMM Opt. §1-§7)            */
  GP_KERNEL_SPLITK = 2,  /* small-M kernel: waves of a workgroup split K,
                            reduced through LDS (for the memory-bound small
                            batch of GEMM Opt. §1.3 / §8.3)                      */
  GP_KERNEL_WIDE = 3     /* 256x256 tiles, 8 waves, A and B both through LDS
                            (INT8, FP8, BF16, FP16; M and N at least 256)        */
};

/* Tuning options. Pass NULL, or a zero-filled struct, for all-automatic;
 * a zero field means "planner's choice". tile_k is in ELEMENTS (as on the
 * pages). For the split-K kernel tile_m is 16, 32 or 64 (16-row blocks per
 * workgroup; 64 runs on 8 waves unless waves says otherwise), tile_n is
 * 16 * (column blocks per workgroup) and tile_k is the K chunk each wave
 * loads per step. A tile that is not compiled into the library is
 * GP_ESHAPE. */
typedef struct gemm_opts {
  int tile_m, tile_n, tile_k;
  int epilogue;     /* GP_EPI_*                                          */
  int kernel;       /* GP_KERNEL_*                                       */
  int xcd_swizzle;  /* 0 auto, 1 XCD-aware grouped tile order, 2 linear  */
  int waves;        /* split-K kernel: waves per workgroup (0 auto); tile
                       kernel: 4, or 8 = two groups of 4 waves that split the
                       K tiles and add their results (where compiled)      */
  int mfma;         /* tile kernel: MFMA block 16 (16x16) or 32 (32x32), 0 auto */
  int pipeline;     /* tile kernel: 1 A staged through VGPRs (2 stages), 2 .. 6 A
                       by LDS DMA with that many stages (where compiled), 0 auto */
  int ksplit;       /* tile kernel: K split across workgroups (GEMM Optimization
                       Guide §13, tiling checklist: enough workgroups to fill
                       the GPU): 0 the planner's
                       choice (no split outside gemm_ex_ws), 1 no split, S = 2 ..
                       64 workgroups per tile, each taking 1/S of the K tiles
                       (S must divide them); S > 1 only through gemm_ex_ws   */
  int scheduler;    /* tile kernel hot-loop schedule (Kernel Tuning Guide §5,
                       GEMM Optimization Guide §5.3): 0 the planner's choice,
                       1 on (loads and LDS reads pinned between the MFMA groups),
                       2 off (the compiler orders the loop); "off" exists for
                       the tiles listed with a scheduler-off variant, with the
                       plain epilogue only (with a bias or an activation:
                       GP_ESHAPE)                                              */
} gemm_opts;

/* What the planner chose (host-side query, no GPU needed). */
typedef struct gemm_plan_info {
  int kernel;
  int tile_m, tile_n, tile_k;       /* tile_k in elements                       */
  int epilogue;
  int xcd_swizzle;                  /* 1 XCD-aware, 2 linear                    */
  int waves;                        /* waves per workgroup                      */
  int threads;                      /* per workgroup                            */
  int lds_bytes;                    /* static LDS per workgroup (without a fused
                                       epilogue; with one, + 4 * tile_n)        */
  int64_t grid;                     /* workgroups                               */
  int64_t k_tiles;                  /* K tiles per workgroup (tile kernel)      */
  int64_t mfma_per_wave_tile;       /* MFMA instructions per wave per K tile    */
  int64_t mfma_total;               /* MFMA instructions the launch issues      */
  int mfma;                         /* MFMA block: 16 (16x16) or 32 (32x32)     */
  int pipeline;                     /* 1 VGPR-staged A; 2 .. 6 LDS DMA stages   */
  int ksplit;                       /* workgroups per tile along K (1: no split)*/
  int scheduler;                    /* 1 pinned hot-loop schedule, 2 compiler's */
  int64_t workspace_bytes;          /* device workspace the call needs (0: none)*/
} gemm_plan_info;

/*
 * gemm_preshuffle_b -- B preshuffle pass (GEMM Optimization Guide §1.4, §12.1).
 *
 * Permutes the bytes of B ([N][Kb] row-major, Kb = K * element bytes) into
 * the layout [N/16][Kb/64][4][16][16 bytes]:
 *     b_shuf[(((n0*(Kb/64) + k0)*4 + g)*16 + j)*16 + b] = B[16*n0 + j][64*k0 + 16*g + b]
 * so that one wave loads a 16-column x 64-byte block as one contiguous KiB,
 * lane 16*g + j taking one dwordx4. The pages run this once on the CPU; here
 * it is a device kernel, run once per B and amortised over GEMM calls.
 *   b       device, [N][Kb] bytes, read only.
 *   b_shuf  device, N*Kb bytes, written; must not overlap b.
 *   dtype   GP_I8, GP_FP8_E4M3, GP_BF16, GP_F16, GP_FP4_E2M1 or GP_I4 (fixes
 *           Kb; MXFP4 block scales are NOT shuffled and stay [N][K/32]).
 *           GP_I4 (W4A8 weights) also reorders the nibbles of every 16-byte
 *           piece: element t of the piece's 32 goes to byte t % 16, the low
 *           nibble for t < 16 and the high nibble otherwise, so that a lane
 *           widens its piece to two int8 operands with masks alone.
 * Requires N % 16 == 0, Kb % 64 == 0 (GP_ESHAPE), N*Kb < 2^31.
 */
int gemm_preshuffle_b(const void* b, void* b_shuf, int64_t N, int64_t K, int dtype, void* stream);

/*
 * gemm_a8w8 -- INT8 or FP8 GEMM on preshuffled B.
 *   a        device, [M][K] int8 / E4M3 codes.
 *   b_shuf   device, output of gemm_preshuffle_b for the same in_dtype.
 *   scale_a  device fp32 [M] or NULL; scale_b device fp32 [N] or NULL.
 *   c        device [M][N]: int32 (out_dtype GP_I32) or bf16 (GP_BF16).
 * Dtype pairs: in GP_I8 -> out GP_I32 with both scales NULL (exact integer
 * accumulation); in GP_FP8_E4M3 -> out GP_BF16 with both scales given:
 *     C[m][n] = bf16_rne((acc[m][n] * scale_a[m]) * scale_b[n]),
 * acc accumulated in fp32 (GEMM Optimization Guide §7.1). Anything else is
 * GP_EDTYPE. The chosen tile_k must divide K (GP_ESHAPE).
 */
int gemm_a8w8(const void* a, const void* b_shuf, const float* scale_a, const float* scale_b,
              void* c, int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
              const gemm_opts* opts, void* stream);

/*
 * gemm_bf16 -- BF16 GEMM on preshuffled B, fp32 accumulation, bf16 output
 * rounded to nearest even (GEMM Optimization Guide §6.2, §7).
 *   a [M][K] bf16, b_shuf from gemm_preshuffle_b(GP_BF16), c [M][N] bf16.
 */
int gemm_bf16(const void* a, const void* b_shuf, void* c, int64_t M, int64_t N, int64_t K,
              const gemm_opts* opts, void* stream);

/*
 * gemm_mxfp4 -- MXFP4 GEMM with gfx950 scaled MFMA (GEMM Optimization Guide
 * §1.3 FP4 row, §6.2, §8.2).
 *   a        device [M][K/2] bytes of E2M1 pairs.
 *   scale_a  device [M][K/32] E8M0 bytes, row-major.
 *   b_shuf   from gemm_preshuffle_b(GP_FP4_E2M1) of B [N][K/2].
 *   scale_b  device [N][K/32] E8M0 bytes, row-major (not shuffled).
 *   c        device [M][N] bf16:
 *     C[m][n] = bf16_rne(sum_k e2m1(A[m][k]) 2^(sa[m][k/32]-127) e2m1(B[n][k]) 2^(sb[n][k/32]-127))
 * with fp32 accumulation. K % 128 == 0.
 */
int gemm_mxfp4(const void* a, const uint8_t* scale_a, const void* b_shuf, const uint8_t* scale_b,
               void* c, int64_t M, int64_t N, int64_t K, const gemm_opts* opts, void* stream);

/*
 * gemm_f16 -- FP16 GEMM on preshuffled B (GEMM Optimization Guide §6.2, f16
 * instruction), fp32 accumulation, fp16 output rounded to nearest even.
 *   a [M][K] fp16, b_shuf from gemm_preshuffle_b(GP_F16), c [M][N] fp16.
 */
int gemm_f16(const void* a, const void* b_shuf, void* c, int64_t M, int64_t N, int64_t K,
             const gemm_opts* opts, void* stream);

/*
 * gemm_w4a8 -- INT4 weights with int8 activations (GEMM Optimization Guide
 * §8.2, INT4 bytes formula): half the weight bytes of INT8 in the
 * memory-bound small-M regime.
 *   a        device [M][K] int8.
 *   b_shuf   from gemm_preshuffle_b(GP_I4) of B [N][K/2] packed INT4.
 *   scale_a  device fp32 [M]; scale_b device fp32 [N] (both required).
 *   c        device [M][N] bf16:
 *     C[m][n] = bf16_rne((acc[m][n] * scale_a[m]) * scale_b[n]),
 * acc = sum_k A[m][k] B[n][k] exact in int32. K % 128 == 0 and K <= 65536.
 * M <= 64, and larger M on small outputs (M * N <= 2^19; with a workspace
 * also M * N * K <= 2^31), run on the small-M kernel (GP_KERNEL_SPLITK: 4
 * or 8 waves split K where their share divides into whole chunks, one wave
 * otherwise); other shapes on the tile kernel, which widens each INT4 piece
 * of B to int8 in registers for two int8 MFMAs.
 */
int gemm_w4a8(const void* a, const void* b_shuf, const float* scale_a, const float* scale_b, void* c,
              int64_t M, int64_t N, int64_t K, const gemm_opts* opts, void* stream);

/*
 * gemm_ex -- any input type, with the fused epilogue of the Kernel Tuning
 * Guide §6 (bias, bias+ReLU, bias+SiLU, bias+GELU).
 *   in_dtype / out_dtype  GP_I8 -> GP_I32, GP_FP8_E4M3 -> GP_BF16,
 *                         GP_BF16 -> GP_BF16, GP_F16 -> GP_F16,
 *                         GP_FP4_E2M1 -> GP_BF16, GP_I4 -> GP_BF16;
 *                         any other pair is GP_EDTYPE.
 *   a, b_shuf, c, scales  as in the type's own entry point (FP8 / W4A8: fp32
 *                         [M] and [N]; MXFP4: E8M0 [M][K/32] and [N][K/32];
 *                         BF16 / FP16 / INT8: both NULL, else GP_EDTYPE).
 *   bias                  device fp32 [N] or NULL (no bias).
 *   act                   GP_ACT_* (GP_EINVAL outside the enum).
 * Floating-point outputs:  C[m][n] = round(act(y[m][n] + bias[n])), y the
 * scaled fp32 accumulator of the type's own entry point, round = RNE to
 * the output type. The INT8 -> int32 path takes neither bias nor
 * activation (GP_EDTYPE).
 */
int gemm_ex(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
            const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
            const gemm_opts* opts, void* stream);

/*
 * gemm_plan -- host-only: validate a problem and report the plan a GEMM
 * call with the same arguments would launch (tile, kernel, grid, LDS, MFMA
 * counts). in_dtype is GP_I8, GP_FP8_E4M3, GP_BF16, GP_F16, GP_FP4_E2M1 or
 * GP_I4 (W4A8). mfma_total counts the MFMAs the launch issues (edge tiles
 * included); it is the problem's (M/ms)(N/ms)(K/K_instr) when the tile
 * divides M and N. Touches
 * no device. Returns the same status the GEMM call would return for these
 * sizes and options (before the device checks).
 */
int gemm_plan(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* opts,
              gemm_plan_info* out);

/*
 * gemm_ex_ws -- gemm_ex with a caller-provided device workspace, which lets
 * the planner split K across workgroups on the tile kernel where the tiles
 * alone would leave CUs idle (GEMM Optimization Guide §13, the tiling item of
 * its checklist: the grid must give the GPU enough workgroups; §1.3's tile
 * table read with the 256 CUs of MI355X); for BF16 / FP16 with long K, where
 * the split lets a larger tile (fewer operand bytes per FLOP) fill the GPU
 * instead of a smaller one; and for 16 to 64 rows with long K, where 16 x 64
 * tiles split along K replace the small-M kernel (FP8 from 8192 bytes per B
 * row, INT8 / BF16 / FP16 / W4A8 from 16384; not MXFP4) if they cut the
 * bytes the busiest CU reads enough to pay for the split.
 *   workspace        device, 16-byte aligned, at least gemm_workspace_size
 *                    bytes for the same arguments (ignored, and may be NULL,
 *                    when that size is 0). Its first 64 KiB hold one arrival
 *                    counter per output tile (a split plan has at most 16384
 *                    tiles, else GP_ESHAPE); the partial sums (fp32, or int32
 *                    for INT8 / W4A8) of every workgroup of each tile follow.
 *                    The first 64 KiB must be ZERO before the first call that
 *                    uses the workspace (e.g. hipMemset it once after
 *                    allocating it); every call leaves them zero again, so
 *                    the same workspace serves any number of later calls, of
 *                    any shapes, that are ordered on one stream. Calls that
 *                    may run at the same time need workspaces of their own.
 *   workspace_bytes  its size in bytes.
 * The workgroups of one tile each add up a contiguous range of the K tiles
 * and store their partial sums; the last of them to finish adds the partial
 * sums in the fixed order of the ranges (so the result is the same on every
 * run, whichever finishes last) and applies the epilogue of gemm_ex. No
 * workgroup waits for another. Other arguments, results and errors as
 * gemm_ex; GP_EWORKSPACE when the workspace is missing or too small.
 */
int gemm_ex_ws(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
               const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
               const gemm_opts* opts, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_ex_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gemm_ex_ws with the library's own workspace instead of the
 * caller's. That workspace is one static device array of
 * GEMM_NOALLOC_SCRATCH_BYTES (32 MiB + 64 KiB) per device, which each device
 * that runs the library holds until the process ends; the call allocates
 * nothing. Its first call on a device looks up the array's device address
 * and clears its counter area with a fill kernel on `stream`; every call
 * leaves the counters zero again. Plans whose workspace would exceed the
 * array (gemm_workspace_size > GEMM_NOALLOC_SCRATCH_BYTES) are GP_EWORKSPACE:
 * call gemm_ex_ws with a workspace of that size instead. Every call on one
 * device shares that device's array, so calls that may overlap in time on
 * one device (on different streams without an ordering between them, or from
 * several host threads at once) race and give wrong results; calls ordered
 * on one stream are safe. Arguments, results and other errors as gemm_ex_ws.
 */
#define GEMM_NOALLOC_SCRATCH_BYTES ((32u << 20) + (64u << 10))
int gemm_ex_noalloc(int in_dtype, int out_dtype, const void* a, const void* b_shuf, const void* scale_a,
                    const void* scale_b, const float* bias, int act, void* c, int64_t M, int64_t N, int64_t K,
                    const gemm_opts* opts, void* stream);

/*
 * gemm_workspace_size -- host-only: the workspace bytes (*bytes) a gemm_ex_ws
 * call with these sizes and options needs; 0 when its plan does not split K
 * across workgroups. Returns the status the planner would (no device check).
 */
int gemm_workspace_size(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* opts, size_t* bytes);

/*
 * gemm_plan_ws -- host-only: as gemm_plan, for the plan of gemm_ex_ws (which
 * may split K across workgroups; out->ksplit, out->workspace_bytes).
 * gemm_plan itself reports the plan of the entry points without a workspace.
 */
int gemm_plan_ws(int in_dtype, int64_t M, int64_t N, int64_t K, const gemm_opts* opts, gemm_plan_info* out);

/* Static, human-readable description of a gp_status value. */
const char* gemm_status_string(int status);

/*
 * Name of the HIP status behind the last GP_EHIP of the calling thread
 * ("hipSuccess" when the library's last HIP call in this thread succeeded).
 * Static string; thread-local state. Each launch clears HIP's per-thread last
 * error right before it, so a GP_EHIP reports the launch's own status, not
 * one left by an earlier runtime call of the caller.
 */
const char* gemm_last_hip_error(void);

/*
 * The runtime call behind the last GP_EHIP of the calling thread: "hipGetDevice"
 * or "hipGetDeviceProperties" (the device check before the first launch on a
 * device), "kernel launch", or "scratch set-up (...)" (gemm_ex_noalloc's first
 * call on a device); "" when the library's last HIP call in this thread
 * succeeded. Static string; thread-local state.
 */
const char* gemm_last_hip_call(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_PRESHUFFLE_H */
