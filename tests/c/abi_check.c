/*
 * abi_check.c -- drives libparallax.so through its C ABI from plain C99, with
 * the HIP runtime's C API for device memory and a stream (no Python, no
 * torch).  The test that runs it (tests/test_gpu_c_abi.py) writes the seeded
 * inputs as raw little-endian bf16 files, runs this program, and compares the
 * output file with the fp64 oracle.
 *
 *   abi_check decode  DIR B Hq Hkv L d      contiguous cache k, v [B, Hkv, L, d]
 *   abi_check ragged  DIR B Hq Hkv L d      packed slabs; DIR/cu.bin holds the
 *                                           B + 1 int64 offsets; L = max context
 *   abi_check prefill DIR B Hq Hkv T d      causal prefill
 *
 * Inputs DIR/q.bin, k.bin, v.bin, rho.bin; output DIR/out.bin.  Also checks
 * that rejected calls return their status codes.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "parallax.h"

static int fail(const char *what, const char *detail) {
    fprintf(stderr, "abi_check: %s: %s\n", what, detail);
    return 1;
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    void *buf = malloc(bytes ? bytes : 1);
    const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(buf);
        return NULL;
    }
    return buf;
}

static int write_file(const char *dir, const char *name, const void *data, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 1;
    const size_t put = fwrite(data, 1, bytes, f);
    return fclose(f) != 0 || put != bytes;
}

/* Host buffer -> new device buffer. */
static void *to_device(const void *host, size_t bytes) {
    void *dev = NULL;
    if (hipMalloc(&dev, bytes ? bytes : 16) != hipSuccess) return NULL;
    if (bytes && hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return dev;
}

int main(int argc, char **argv) {
    if (argc != 8) return fail("usage", "abi_check decode|ragged|prefill DIR B Hq Hkv N d");
    const char *mode = argv[1], *dir = argv[2];
    const int32_t B = atoi(argv[3]), Hq = atoi(argv[4]), Hkv = atoi(argv[5]), d = atoi(argv[7]);
    const int64_t N = atoll(argv[6]);
    const int is_decode = strcmp(mode, "decode") == 0, is_ragged = strcmp(mode, "ragged") == 0;
    const int is_prefill = strcmp(mode, "prefill") == 0;
    if (!is_decode && !is_ragged && !is_prefill) return fail("mode", mode);

    const float scale = 1.0f / sqrtf((float)d);
    const size_t e = sizeof(uint16_t); /* bf16 */
    int64_t *cu = NULL;
    size_t kv_rows;
    if (is_ragged) {
        cu = read_file(dir, "cu.bin", (size_t)(B + 1) * sizeof(int64_t));
        if (!cu) return fail("read", "cu.bin");
        kv_rows = (size_t)cu[B];
    } else {
        kv_rows = (size_t)B * (size_t)N;
    }
    const size_t q_elems = (size_t)B * Hq * d * (is_prefill ? (size_t)N : 1);
    const size_t kv_elems = kv_rows * Hkv * d;

    void *hq = read_file(dir, "q.bin", q_elems * e), *hr = read_file(dir, "rho.bin", q_elems * e);
    void *hk = read_file(dir, "k.bin", kv_elems * e), *hv = read_file(dir, "v.bin", kv_elems * e);
    if (!hq || !hr || !hk || !hv) return fail("read", "q/k/v/rho.bin");

    void *q = to_device(hq, q_elems * e), *rho = to_device(hr, q_elems * e);
    void *k = to_device(hk, kv_elems * e), *v = to_device(hv, kv_elems * e);
    void *out = NULL, *cu_dev = NULL, *ws = NULL;
    if (!q || !rho || !k || !v || hipMalloc(&out, q_elems * e) != hipSuccess)
        return fail("hip", "device allocation or copy");
    if (is_ragged && !(cu_dev = to_device(cu, (size_t)(B + 1) * sizeof(int64_t))))
        return fail("hip", "cu_seqlens copy");

    hipStream_t stream;
    if (hipStreamCreate(&stream) != hipSuccess) return fail("hip", "stream");

    /* Rejected calls: checked on the host, nothing reaches the device. */
    if (parallax_fwd_prefill(q, k, v, rho, out, B, Hq, Hkv, 16, 80, scale, PLX_DTYPE_BF16, stream) !=
        PLX_ERR_UNSUPPORTED)
        return fail("status", "head dim 80 must be PLX_ERR_UNSUPPORTED");
    if (parallax_fwd_prefill(q, k, v, rho, NULL, B, Hq, Hkv, 16, d, scale, PLX_DTYPE_BF16, stream) !=
        PLX_ERR_INVALID_ARGUMENT)
        return fail("status", "null out must be PLX_ERR_INVALID_ARGUMENT");

    plx_status_t st;
    if (is_prefill) {
        st = parallax_fwd_prefill(q, k, v, rho, out, B, Hq, Hkv, (int32_t)N, d, scale, PLX_DTYPE_BF16, stream);
    } else {
        const size_t ws_bytes = parallax_fwd_decode_workspace_size(B, Hq, Hkv, d, N, PLX_DTYPE_BF16);
        if (ws_bytes == (size_t)-1) return fail("status", "workspace size query rejected the shape");
        if (ws_bytes && hipMalloc(&ws, ws_bytes) != hipSuccess) return fail("hip", "workspace");
        if (ws_bytes && parallax_fwd_decode(q, rho, k, v, cu_dev, N, out, B, Hq, Hkv, d, scale,
                                            PLX_DTYPE_BF16, ws, ws_bytes - 1, stream) !=
                            PLX_ERR_WORKSPACE_TOO_SMALL)
            return fail("status", "short workspace must be PLX_ERR_WORKSPACE_TOO_SMALL");
        st = parallax_fwd_decode(q, rho, k, v, cu_dev, N, out, B, Hq, Hkv, d, scale, PLX_DTYPE_BF16, ws,
                                 ws_bytes, stream);
    }
    if (st != PLX_OK) return fail("call", parallax_status_string(st));
    if (hipStreamSynchronize(stream) != hipSuccess) return fail("hip", "stream synchronize");

    void *hout = malloc(q_elems * e);
    if (!hout || hipMemcpy(hout, out, q_elems * e, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hip", "copy of the output");
    if (write_file(dir, "out.bin", hout, q_elems * e)) return fail("write", "out.bin");

    hipFree(q);
    hipFree(rho);
    hipFree(k);
    hipFree(v);
    hipFree(out);
    if (cu_dev) hipFree(cu_dev);
    if (ws) hipFree(ws);
    hipStreamDestroy(stream);
    free(hq);
    free(hr);
    free(hk);
    free(hv);
    free(hout);
    free(cu);
    printf("abi_check %s: ok\n", mode);
    return 0;
}
