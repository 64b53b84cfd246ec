"""fp64 CPU oracle for paged GQA decode attention -- test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. It shares no code with the GPU library.
"""
