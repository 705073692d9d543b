/*
 * nvfp4_probe.h -- C ABI of the measurement and test probes that ship beside
 * the NVFP4 decode-projection library (lib/libnvfp4_probe.so).  They are not
 * part of the projection path: nothing in libnvfp4.so calls them.
 *
 * Read-stream probe.  A small-M decode projection is one streaming read of
 * the packed weights (ReSET project page, "Why a CUDA-core NVFP4 kernel?":
 * the gain comes from moving fewer weight bytes), so the fastest plain read
 * of the same number of bytes on the same GPU is the ceiling a GEMV can
 * reach there.  nvfp4_probe_read reads `bytes` bytes at `buf` once, folding
 * them into an XOR so that no load can be dropped:
 *   - the buffer is cut into `grid` contiguous slices of whole 16-byte units,
 *     one per workgroup of 256 threads;
 *   - variants "vgpr_u<U>_<NT>": every lane keeps U 16-byte buffer loads in
 *     flight in registers (NT = 1: with the non-temporal hint);
 *   - variants "lds_d<D>": each wave streams 1 KB chunks straight into an LDS
 *     ring of D slots (direct-to-LDS buffer loads) and reads them back.
 * `sink` (device, >= grid uint32) is written only when a slice's XOR equals
 * a fixed constant, so it normally receives nothing.  Device pointers are
 * the caller's; work is enqueued on `stream` (a hipStream_t as void*).
 *
 * Converter probe.  nvfp4_probe_convert runs, over n inputs, one of the
 * gfx950 conversion instructions the NVFP4 kernels use, so that a test can
 * compare every code with the exact format decode (ReSET reading notes,
 * section 2.1: E2M1 elements, E4M3 block scales):
 *   NVFP4_PROBE_FP4_TO_F16   in[i] = 8 E2M1 codes; out[4i + b] = the f16 pair
 *                            of byte b (low nibble in the low half), scale 1
 *   NVFP4_PROBE_FP4_TO_F32   the same to f32: out[8i + 2b], out[8i + 2b + 1]
 *   NVFP4_PROBE_FP8_TO_F32   in[i] = 4 E4M3 codes; out[4i + 0..3] = the four
 *                            values as f32 (bytes 0..3)
 *   NVFP4_PROBE_F32_TO_FP4   in[2i], in[2i+1] = two f32 bit patterns;
 *                            out[i] = the byte of their two E2M1 codes (first
 *                            in the low nibble), scale 1
 *   NVFP4_PROBE_F16_SCALE_MUL in[2i], in[2i+1] = two f16 pairs; out[i] = their
 *                            packed f16 product
 * Buffers: in and out are device arrays of uint32 of the sizes above.
 *
 * Every call validates on the host and returns a negative status without
 * launching when an argument is out of range.
 */
#ifndef NVFP4_PROBE_H
#define NVFP4_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { NVFP4_PROBE_OK = 0, NVFP4_PROBE_ERR_ARG = -1, NVFP4_PROBE_ERR_HIP = -2 };

enum {
  NVFP4_PROBE_FP4_TO_F16 = 0,
  NVFP4_PROBE_FP4_TO_F32 = 1,
  NVFP4_PROBE_FP8_TO_F32 = 2,
  NVFP4_PROBE_F32_TO_FP4 = 3,
  NVFP4_PROBE_F16_SCALE_MUL = 4
};

/* Number of read-probe variants, and the name of variant i (NULL past the end). */
int nvfp4_probe_read_count(void);
const char* nvfp4_probe_read_name(int variant);

/* One read of buf[0, bytes) (16-byte aligned, bytes % 16 == 0, each slice
 * under 2 GB) with `grid` workgroups (1 .. 2^20). */
int nvfp4_probe_read(int variant, const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream);

/* An empty kernel of `grid` workgroups of `threads` threads: the launch floor. */
int nvfp4_probe_empty(int grid, int threads, void* stream);

/* Converter probe; n = inputs (pairs for the two-operand ops), 1 .. 2^24. */
int nvfp4_probe_convert(int op, const uint32_t* in, uint32_t* out, int n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_PROBE_H */
