"""fp64 CPU oracle for the Gated DeltaNet state update -- test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package; the GPU library never does.
"""
