/*
 * ssm_roofline.h -- microbenchmarks of the two hardware ceilings the scan
 * kernels of ssm_scan.h are measured against, run by the benchmark in the
 * same process as the kernels it rates.
 *
 * The pages place the cost of the selective scan in data movement between
 * HBM and on-chip memory rather than in arithmetic (the inferownia.pl page
 * on Mamba, section "Cena selekcji": the fused scan keeps the expanded state
 * on chip).  On an MI355X the scan at 16 states needs, per state update, one
 * exponential and about five other fp32 operations, so it can be bound by
 * VALU issue instead: these calls measure both ceilings on the device
 * itself, so that a kernel's time can be stated as a fraction of each.
 * They are not part of the method.
 *
 * Conventions as in ssm_scan.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t, NULL = null stream), all checks
 * before any HIP call, a status return, ssm_last_error() for the message.
 */
#ifndef SSM_ROOFLINE_H
#define SSM_ROOFLINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes per HBM pass must be a multiple of this (one workgroup's span). */
#define SSM_ROOFLINE_HBM_QUANTUM 16384
/* Threads of a VALU pass must be a multiple of this (one workgroup). */
#define SSM_ROOFLINE_VALU_QUANTUM 256

typedef enum {
    SSM_ROOFLINE_COPY = 0,  /* b = a: bytes read and bytes written, 16-byte
                               non-temporal loads and stores */
    SSM_ROOFLINE_RMW = 1,   /* a = a*0.5 + 0.25 in place: the decode step's
                               read-modify-write pattern; b unused (NULL) */
    SSM_ROOFLINE_READ = 2   /* reads a; b: 4 bytes the kernel may write */
} ssm_roofline_hbm_kind;

/* `repeats` passes of one HBM kernel over `bytes` bytes of `a` (and `b`).
 *  a, b     device buffers, 16-byte aligned; for COPY both of `bytes` bytes
 *           and not overlapping; for RMW `a` is modified
 *  bytes    > 0, a multiple of SSM_ROOFLINE_HBM_QUANTUM, below 2^46
 *  repeats  1..1000 */
int ssm_roofline_hbm(int kind, void *a, void *b, size_t bytes, int repeats,
                     void *stream);

typedef enum {
    SSM_ROOFLINE_EXP = 0,   /* chains of v_exp_f32: x = 2^-x */
    SSM_ROOFLINE_FMA = 1,   /* chains of v_fma_f32: x = x*a + b */
    SSM_ROOFLINE_MIXED = 2  /* half of the chains of each kind, interleaved */
} ssm_roofline_valu_kind;

/* One VALU pass: `threads` threads each run `iters` iterations of 8
 * independent dependency chains (8 operations per iteration), then write
 * one float to out[thread].
 *  out      device fp32 buffer of `threads` elements
 *  threads  > 0, a multiple of SSM_ROOFLINE_VALU_QUANTUM, at most 2^26
 *  iters    1..2^20 */
int ssm_roofline_valu(int kind, float *out, int64_t threads, int iters,
                      void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_ROOFLINE_H */
