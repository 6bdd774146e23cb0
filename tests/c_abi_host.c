/*
 * c_abi_host.c -- test program: the library's C boundary used from plain C
 * (no C++, no Python), host-only calls: the ABI version, a query of the
 * decode shape (bf16 experts [256, 1536, 4096], top-8), and a rejected
 * query with its error text.  Prints one line per check.
 */
#include <stdio.h>
#include <string.h>

#include "eidm.h"

int main(void) {
    printf("abi %d\n", eidm_abi_version());
    eidm_shape s;
    memset(&s, 0, sizeof s);
    s.struct_size = sizeof s;
    s.weight_dtype = EIDM_DTYPE_BF16;
    s.m = 1;
    s.n = 1536;
    s.k = 4096;
    s.top_k = 8;
    s.n_experts = 256;
    s.expert_stride_bytes = (uint64_t)1536 * 4096 * 2;
    eidm_requirements r;
    memset(&r, 0, sizeof r);
    r.struct_size = sizeof r;
    int rc = eidm_query(&s, EIDM_ROUTE_AUTO, &r);
    printf("query %d route %d weight_bytes %llu outputs %llu\n", rc, (int)r.route,
           (unsigned long long)r.required_weight_bytes, (unsigned long long)r.output_elements);
    s.k = 0;
    rc = eidm_query(&s, EIDM_ROUTE_AUTO, &r);
    printf("rejected %d %s\n", rc, eidm_last_error());
    return 0;
}
