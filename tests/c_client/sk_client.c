/*
 * A plain C99 client of libsplitkv (include/splitkv.h): it links the shared
 * library by name, allocates device memory with the HIP runtime, runs
 * counts -> partial -> combine on a dense batch read from files, and writes
 * the results back to files for the test suite to compare with the oracle.
 *
 *   sk_client DIR
 *
 * DIR/problem.txt holds "name value" lines: batch heads sq sk dqk dv split
 * npb mask prefix_offset last_valid scale.  DIR/q.bin, k.bin, v.bin hold
 * bf16 tensors [B][H][S][D] (row-major, contiguous).  Written: out.bin (bf16
 * [B][H][Sq][Dv]), lse.bin (f32 [H][B*Sq]) and counts.bin (int32 [B*Sq]).
 * Exit status 0 on success; on failure the library's message is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "splitkv.h"

static int fail_hip(hipError_t e, const char* what) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
}

static int fail_sk(sk_status s, const char* what) {
    fprintf(stderr, "%s: %s (%s)\n", what, sk_status_string(s), sk_last_error());
    return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof(path), "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* buf = malloc(bytes ? bytes : 1);
    const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(buf);
        return NULL;
    }
    return buf;
}

static int write_file(const char* dir, const char* name, const void* data, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof(path), "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const size_t put = fwrite(data, 1, bytes, f);
    fclose(f);
    return put != bytes;
}

/* Copies a host buffer to a new device allocation. */
static int to_device(const void* host, size_t bytes, void** dev) {
    hipError_t e = hipMalloc(dev, bytes ? bytes : 16);
    if (e != hipSuccess) return fail_hip(e, "hipMalloc");
    e = hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice);
    return e == hipSuccess ? 0 : fail_hip(e, "hipMemcpy to device");
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    if (sk_abi_version() != SK_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header %d\n", sk_abi_version(), SK_ABI_VERSION);
        return 1;
    }

    /* the problem */
    long long batch = 0, heads = 0, sq = 0, sk = 0, dqk = 0, dv = 0, split = 0, npb = 0, mask = 0;
    long long prefix_offset = 0, last_valid = -1;
    double scale = 0.0;
    {
        char path[4096], key[64];
        snprintf(path, sizeof(path), "%s/problem.txt", dir);
        FILE* f = fopen(path, "r");
        if (!f) {
            fprintf(stderr, "cannot read %s\n", path);
            return 1;
        }
        double value;
        while (fscanf(f, "%63s %lf", key, &value) == 2) {
            if (!strcmp(key, "batch")) batch = (long long)value;
            else if (!strcmp(key, "heads")) heads = (long long)value;
            else if (!strcmp(key, "sq")) sq = (long long)value;
            else if (!strcmp(key, "sk")) sk = (long long)value;
            else if (!strcmp(key, "dqk")) dqk = (long long)value;
            else if (!strcmp(key, "dv")) dv = (long long)value;
            else if (!strcmp(key, "split")) split = (long long)value;
            else if (!strcmp(key, "npb")) npb = (long long)value;
            else if (!strcmp(key, "mask")) mask = (long long)value;
            else if (!strcmp(key, "prefix_offset")) prefix_offset = (long long)value;
            else if (!strcmp(key, "last_valid")) last_valid = (long long)value;
            else if (!strcmp(key, "scale")) scale = value;
        }
        fclose(f);
    }
    sk_problem p;
    memset(&p, 0, sizeof(p));
    p.batch = (int32_t)batch;
    p.num_heads = (int32_t)heads;
    p.max_seqlen_q = (int32_t)sq;
    p.max_seqlen_k = (int32_t)sk;
    p.head_dim_qk = (int32_t)dqk;
    p.head_dim_v = (int32_t)dv;
    p.split_kv = (int32_t)split;
    p.n_per_block = (int32_t)npb;
    p.mask = (int32_t)mask;
    p.dtype = SK_BF16;
    p.out_dtype = SK_BF16;
    p.prefix_offset = prefix_offset;
    p.last_valid_kv_index = last_valid;
    p.softmax_scale = (float)scale;
    p.window_left = -1;
    /* dense [B][H][S][D], contiguous */
    p.q_stride_row = dqk;
    p.q_stride_head = sq * dqk;
    p.q_stride_batch = heads * sq * dqk;
    p.k_stride_row = dqk;
    p.k_stride_head = sk * dqk;
    p.k_stride_batch = heads * sk * dqk;
    p.v_stride_row = dv;
    p.v_stride_head = sk * dv;
    p.v_stride_batch = heads * sk * dv;
    p.o_stride_row = dv;
    p.o_stride_head = sq * dv;
    p.o_stride_batch = heads * sq * dv;

    const int64_t rows = sk_rows(&p);
    if (rows < 0) return fail_sk(SK_ERR_INVALID_ARG, "sk_rows");
    size_t o_part_bytes = 0, lse_part_bytes = 0;
    sk_status st = sk_workspace_bytes(&p, &o_part_bytes, &lse_part_bytes);
    if (st != SK_OK) return fail_sk(st, "sk_workspace_bytes");
    const int64_t scratch_bytes = sk_partial_scratch_bytes(&p);
    if (scratch_bytes < 0) return fail_sk(SK_ERR_INVALID_ARG, "sk_partial_scratch_bytes");

    /* inputs */
    const size_t q_bytes = (size_t)(batch * heads * sq * dqk) * 2, k_bytes = (size_t)(batch * heads * sk * dqk) * 2;
    const size_t v_bytes = (size_t)(batch * heads * sk * dv) * 2, out_bytes = (size_t)(batch * heads * sq * dv) * 2;
    void* hq = read_file(dir, "q.bin", q_bytes);
    void* hk = read_file(dir, "k.bin", k_bytes);
    void* hv = read_file(dir, "v.bin", v_bytes);
    if (!hq || !hk || !hv) {
        fprintf(stderr, "cannot read q.bin / k.bin / v.bin of the expected sizes\n");
        return 1;
    }
    void *q, *k, *v, *o_part, *lse_part, *counts, *out, *lse_out, *scratch = NULL;
    if (to_device(hq, q_bytes, &q) || to_device(hk, k_bytes, &k) || to_device(hv, v_bytes, &v)) return 1;
    hipError_t e;
    if ((e = hipMalloc(&o_part, o_part_bytes)) != hipSuccess || (e = hipMalloc(&lse_part, lse_part_bytes)) ||
        (e = hipMalloc(&counts, (size_t)rows * 4)) || (e = hipMalloc(&out, out_bytes)) ||
        (e = hipMalloc(&lse_out, (size_t)(heads * rows) * 4)))
        return fail_hip(e, "hipMalloc");
    if (scratch_bytes > 0 && (e = hipMalloc(&scratch, (size_t)scratch_bytes)) != hipSuccess)
        return fail_hip(e, "hipMalloc");
    p.partial_scratch = scratch;
    p.partial_scratch_bytes = scratch_bytes;

    /* the forward pass on a stream of our own */
    hipStream_t stream;
    if ((e = hipStreamCreate(&stream)) != hipSuccess) return fail_hip(e, "hipStreamCreate");
    if ((st = sk_valid_split_counts(&p, (int32_t*)counts, (void*)stream)) != SK_OK) return fail_sk(st, "counts");
    if ((st = sk_attn_partial(&p, q, k, v, (float*)o_part, (float*)lse_part, (void*)stream)) != SK_OK)
        return fail_sk(st, "partial");
    if ((st = sk_attn_combine(&p, (const float*)o_part, (const float*)lse_part, (const int32_t*)counts, out,
                              (float*)lse_out, (void*)stream)) != SK_OK)
        return fail_sk(st, "combine");
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");

    /* an invalid call is refused with a message and enqueues nothing */
    {
        sk_problem bad = p;
        bad.split_kv = -1;
        if (sk_attn_partial(&bad, q, k, v, (float*)o_part, (float*)lse_part, (void*)stream) != SK_ERR_INVALID_ARG ||
            sk_last_error()[0] == '\0') {
            fprintf(stderr, "an invalid split_kv was not refused\n");
            return 1;
        }
    }

    /* results */
    void* hout = malloc(out_bytes ? out_bytes : 1);
    void* hlse = malloc((size_t)(heads * rows) * 4 + 1);
    void* hcounts = malloc((size_t)rows * 4 + 1);
    if (!hout || !hlse || !hcounts) return 1;
    if ((e = hipMemcpy(hout, out, out_bytes, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(hlse, lse_out, (size_t)(heads * rows) * 4, hipMemcpyDeviceToHost)) ||
        (e = hipMemcpy(hcounts, counts, (size_t)rows * 4, hipMemcpyDeviceToHost)))
        return fail_hip(e, "hipMemcpy to host");
    if (write_file(dir, "out.bin", hout, out_bytes) || write_file(dir, "lse.bin", hlse, (size_t)(heads * rows) * 4) ||
        write_file(dir, "counts.bin", hcounts, (size_t)rows * 4)) {
        fprintf(stderr, "cannot write the results\n");
        return 1;
    }
    (void)hipStreamDestroy(stream);
    (void)hipFree(q);
    (void)hipFree(k);
    (void)hipFree(v);
    (void)hipFree(o_part);
    (void)hipFree(lse_part);
    (void)hipFree(counts);
    (void)hipFree(out);
    (void)hipFree(lse_out);
    if (scratch) (void)hipFree(scratch);
    free(hq);
    free(hk);
    free(hv);
    free(hout);
    free(hlse);
    free(hcounts);
    printf("sk_client: ok (%lld rows)\n", (long long)rows);
    return 0;
}
